// skv_decode_step_static: skv_decode_step with its scratch memory (the score
// row and the split-K partial states) taken from a fixed device array of the
// library instead of caller buffers, for callers that cannot allocate.
//
// The array lives in this code object, one copy per GPU, from the first call
// on that device until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device copy: its device address is looked up
// once per device with hipGetSymbolAddress (that device current) and only
// that address is ever handed to kernels.  No call here allocates memory.
#include <hip/hip_runtime.h>

#include <mutex>

#include "skv.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB per GPU
constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

size_t round_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Device address of this GPU's scratch array (looked up on first use).
skv_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SKV_EDEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SKV_EDEVICE;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return SKV_OK;
}

}  // namespace

extern "C" {

size_t skv_static_scratch_bytes(void) { return kScratchBytes; }

skv_status skv_decode_step_static(const skv_cache* c, const int32_t* pos0, const void* k_new,
                                  const void* v_new, int32_t src_dtype, const float* q,
                                  int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                  const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                                  int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                                  float softmax_scale, int32_t n_split, float* out,
                                  hipStream_t stream) {
  if (c == nullptr) return SKV_EINVAL;
  const size_t ws = skv_workspace_bytes(c->batch, n_heads, c->head_dim, n_split);
  if (ws == 0) return SKV_EINVAL;
  const int32_t max_blocks = skv_max_blocks(c);
  const size_t score_bytes =
      k_sel != nullptr ? round_up(sizeof(float) * size_t(c->batch) * size_t(c->n_kv_heads) *
                                  size_t(max_blocks))
                       : 0;
  if (score_bytes + ws > kScratchBytes) return SKV_ERANGE;
  void* base = nullptr;
  const skv_status st = scratch_ptr(&base);
  if (st != SKV_OK) return st;
  unsigned char* b = static_cast<unsigned char*>(base);
  float* score = k_sel != nullptr ? reinterpret_cast<float*>(b) : nullptr;
  void* workspace = b + score_bytes;
  // every byte of the scratch that is read in a call is first written in
  // that call (scores by the bounds pass, partial states by the attention
  // parts), so nothing needs clearing between calls
  return skv_decode_step(c, pos0, k_new, v_new, src_dtype, q, n_heads, seq_len, max_len, k_sel,
                         n_sink, n_recent, max_sel, score, sel_idx, sel_cnt, softmax_scale,
                         n_split, workspace, ws, out, stream);
}

}  // extern "C"
