// The split workspace cache: one f32 buffer per (device, stream) for the
// kernels that reduce partial results in a second pass (the prefill kernel's K
// splits and the few-row kernel's K chunks), bounded and releasable.
//
// Calls on one stream are ordered, so they may share its buffer; calls on
// different streams use different buffers.  A call that needs more than its
// stream's buffer holds grows it.  Buffers come from hipMalloc and go back
// with hipFree, which waits for the device to finish the work already
// enqueued; so a buffer is never freed ahead of a kernel that uses it, even
// when the stream it was cached for has since been destroyed.  At most
// kMaxEntries streams per device keep a buffer: the least recently used one is
// released to make room.  mxq_release_workspaces() releases them all.
//
// The mutex is held from split_workspace_locked() until the caller has
// enqueued the kernels that use the buffer, so another thread cannot free it
// in between.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <list>
#include <mutex>

#include "../../include/mxq.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

struct Entry {
  int device;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};

std::mutex g_ws_mu;
std::list<Entry>* g_ws = nullptr;  // most recently used first

void free_entry(const Entry& e) {
  int cur = -1;
  const bool restore = hipGetDevice(&cur) == hipSuccess && cur != e.device;
  if (restore) (void)hipSetDevice(e.device);
  (void)hipFree(e.ptr);
  if (restore) (void)hipSetDevice(cur);
  (void)hipGetLastError();
}

}  // namespace

std::mutex& split_workspace_mutex() { return g_ws_mu; }

float* split_workspace_locked(int device, hipStream_t stream, size_t bytes) {
  if (!g_ws) g_ws = new std::list<Entry>();
  for (auto it = g_ws->begin(); it != g_ws->end(); ++it) {
    if (it->device != device || it->stream != stream) continue;
    if (it->bytes >= bytes) {
      g_ws->splice(g_ws->begin(), *g_ws, it);  // most recently used
      return static_cast<float*>(g_ws->front().ptr);
    }
    free_entry(*it);  // too small: replaced by a larger one below
    g_ws->erase(it);
    break;
  }
  int per_device = 0;
  for (const Entry& e : *g_ws) per_device += e.device == device;
  if (per_device >= kWorkspaceEntries) {
    for (auto it = g_ws->end(); it != g_ws->begin();) {
      --it;
      if (it->device == device) {  // the least recently used of this device
        free_entry(*it);
        g_ws->erase(it);
        break;
      }
    }
  }
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_ws->push_front(Entry{device, stream, p, bytes});
  return static_cast<float*>(p);
}

size_t split_workspace_cached_bytes(int device) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  size_t total = 0;
  if (g_ws)
    for (const Entry& e : *g_ws) total += e.device == device ? e.bytes : 0;
  return total;
}

int split_workspace_release_all() {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  int n = 0;
  if (g_ws) {
    for (const Entry& e : *g_ws) {
      free_entry(e);
      ++n;
    }
    g_ws->clear();
  }
  return n;
}

}  // namespace mxq
