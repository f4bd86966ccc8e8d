// ds_rows_indexer_topk_attn_noalloc: the one-call decode core with its two
// workspaces carved out of a device array the library owns, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid allocation).
//
// The array `scratch` is a file-scope __device__ object: every GPU the
// library runs on holds its own copy, for the life of the process. In host
// code its name is only a host-side stand-in, so the device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// kept per device; only that address is handed to the kernels. The call
// allocates nothing and frees nothing; it rejects work whose workspaces do
// not fit the array. Calls that overlap on one GPU (e.g. on two streams)
// share the array and race: serialise them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ds_rows.h"
#include "ds_rows_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[DS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device, once taken

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// The current device's address of `scratch` (set up on the first call on
// that device), or nullptr with the error recorded.
void *device_scratch(ds_status *st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = ds::record_error(DS_ERR_DEVICE, "no current HIP device for the scratch array");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *st = ds::record_error(DS_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  *st = DS_OK;
  return g_scratch[dev];
}

}  // namespace

extern "C" ds_status ds_rows_indexer_topk_attn_noalloc(
    const ds_indexer_rows *irows, const ds_sparse_rows *srows, const void *idx_q, size_t idx_q_elems,
    const float *weights, size_t weights_elems, float *scores, size_t scores_elems, int32_t *indices,
    size_t indices_elems, const void *q, size_t q_elems, const float *sinks, size_t sinks_elems, float scale,
    float *out, size_t out_elems, void *stream) {
  // The workspace sizes (0 for an invalid table; the query then recorded why).
  const uint64_t idx_bytes = ds_rows_indexer_topk_workspace_bytes(irows);
  if (idx_bytes == 0) return DS_ERR_INVALID_ARGUMENT;
  const uint64_t attn_bytes = ds_rows_attn_workspace_bytes(srows);
  if (attn_bytes == 0) return DS_ERR_INVALID_ARGUMENT;
  const uint64_t need = align256(idx_bytes) + attn_bytes;
  if (need > DS_NOALLOC_SCRATCH_BYTES)
    return ds::record_error(DS_ERR_INVALID_ARGUMENT,
                            "the call needs %llu bytes of workspace; the no-alloc scratch array holds %llu",
                            static_cast<unsigned long long>(need),
                            static_cast<unsigned long long>(DS_NOALLOC_SCRATCH_BYTES));
  ds_status st;
  char *base = static_cast<char *>(device_scratch(&st));
  if (!base) return st;
  // Every other check (operands, the two tables' correspondence, the device)
  // is the one-call entry point's own.
  return ds_rows_indexer_topk_attn(irows, srows, idx_q, idx_q_elems, weights, weights_elems, scores, scores_elems,
                                   base, idx_bytes, indices, indices_elems, q, q_elems, sinks, sinks_elems, scale,
                                   base + align256(idx_bytes), attn_bytes, out, out_elems, stream);
}
