// svd_noalloc.hip -- svd_select_and_verify_noalloc: the select-and-verify call
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// Its workspace is a file-scope device array of SVD_NOALLOC_SCRATCH_BYTES that
// every GPU the library runs on holds until the process ends.  Host code never
// passes the array's name to a kernel or a copy (on the host it names a
// stand-in, not device memory): the first call on a device, with that device
// current, looks up the array's device address with hipGetSymbolAddress and
// keeps it for that device; every call then hands that address to
// svd_select_and_verify as its workspace.  No call allocates or frees.
#include <hip/hip_runtime.h>

#include <mutex>

#include "svd.h"

namespace {

constexpr size_t kScratchBytes = SVD_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void *scratch_addr[kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device.
int scratch_on_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SVD_EHIP;
  std::lock_guard<std::mutex> g(scratch_mu);
  if (!scratch_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SVD_EHIP;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return SVD_OK;
}

}  // namespace

extern "C" int svd_select_and_verify_noalloc(
    const void *p_logits, const void *q_logits, const int32_t *drafts, svd_dtype_t dtype,
    int64_t B, int32_t K, int32_t gamma, int32_t V, float temp_p, float temp_q, uint64_t seed,
    uint64_t row_base, int32_t *selected, int32_t *accept_len, int32_t *next_token,
    float *scores, float *alpha, float *beta, void *hip_stream) {
  // sizes first, on the host: nothing touches the GPU for a call that fails here
  const size_t need = svd_workspace_bytes(B, K, gamma, V);
  if (need == 0) return SVD_EINVAL;
  if (need > kScratchBytes) return SVD_ESCRATCH;
  // every other check too: with a zero-byte workspace (at a fake, never used,
  // aligned address) the checked entry point stops at the workspace's size
  // once the arguments pass, before any HIP call
  const int pre = svd_select_and_verify(p_logits, q_logits, drafts, dtype, B, K, gamma, V, temp_p,
                                        temp_q, seed, row_base, selected, accept_len, next_token,
                                        scores, alpha, beta, reinterpret_cast<void *>(uintptr_t{256}),
                                        0, hip_stream);
  if (pre != SVD_EWORKSPACE) return pre;
  void *ws = nullptr;
  const int rc = scratch_on_current_device(&ws);
  if (rc != SVD_OK) return rc;
  return svd_select_and_verify(p_logits, q_logits, drafts, dtype, B, K, gamma, V, temp_p, temp_q,
                               seed, row_base, selected, accept_len, next_token, scores, alpha,
                               beta, ws, kScratchBytes, hip_stream);
}
