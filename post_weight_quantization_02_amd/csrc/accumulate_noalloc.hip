// gptq_hessian_accumulate_noalloc: H += alpha * X^T X with the split partial
// tiles in a fixed device array instead of a caller workspace, for callers
// that cannot allocate (see include/gptq.h).
//
// The array `scratch` is a file-scope __device__ object: every GPU the
// library runs on holds its own copy from module load until the process
// ends. In host code its name is only a stand-in for that object, so the
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is passed to the kernels.
#include <mutex>

#include "common.h"

namespace {

using namespace gptq;

constexpr size_t kScratchBytes = size_t(96) << 20;
constexpr int64_t kTileBytes = int64_t(kSyrkTile) * kSyrkTile * sizeof(float);
constexpr int64_t kScratchTiles = int64_t(kScratchBytes) / kTileBytes;  // 384
constexpr int64_t kMaxSplitTokens = 4096;  // the split length of the workspace path
constexpr int64_t kMaxSplits = 128;        // the most splits syrk_splits chooses
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch` (nullptr on error).
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" gptq_status gptq_hessian_accumulate_noalloc(float* H, int64_t d, const void* X,
                                                       int64_t n, int64_t ldx, float alpha,
                                                       void* stream) {
  if (d < 1 || d > (1 << 20) || n < 0 || ldx < d) return GPTQ_ERR_INVALID_ARG;
  if (H == nullptr || (n > 0 && X == nullptr)) return GPTQ_ERR_INVALID_ARG;
  if (n > 0 && n > ((int64_t)1 << 40) / ldx) return GPTQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(H) & 3) || (reinterpret_cast<uintptr_t>(X) & 1))
    return GPTQ_ERR_INVALID_ARG;
  const int64_t nb = ceil_div(d, kSyrkTile);
  const int64_t tiles = nb * (nb + 1) / 2;
  if (tiles > kScratchTiles) return GPTQ_ERR_UNSUPPORTED;  // d > 6912
  if (n == 0) return GPTQ_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GPTQ_ERR_HIP;
  if (s != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return GPTQ_ERR_HIP;
    if (sdev != dev) return GPTQ_ERR_INVALID_ARG;  // the stream's device must be current
  }
  float* P = reinterpret_cast<float*>(scratch_address(dev));
  if (P == nullptr) return GPTQ_ERR_HIP;
  // Passes of at most max_splits splits of at most 4096 tokens each: every
  // split is summed as in gptq_hessian_accumulate, and each pass adds its
  // fp64 split sum into H (one fp32 rounding per pass).
  const int64_t max_splits = (kScratchTiles / tiles < kMaxSplits) ? kScratchTiles / tiles
                                                                  : kMaxSplits;
  const _Float16* Xh = reinterpret_cast<const _Float16*>(X);
  for (int64_t t = 0; t < n;) {
    const int64_t n_pass = (n - t < max_splits * kMaxSplitTokens) ? n - t
                                                                   : max_splits * kMaxSplitTokens;
    int splits = syrk_splits(d, n_pass);
    if (splits > max_splits) splits = (int)max_splits;
    const int64_t kper = syrk_kper(n_pass, splits);
    if (kper > kMaxSplitTokens || (int64_t)splits * tiles > kScratchTiles) return GPTQ_ERR_HIP;
    if (launch_syrk_partial(Xh + t * ldx, ldx, (int)d, n_pass, splits, kper, P, s) != hipSuccess)
      return GPTQ_ERR_HIP;
    if (launch_syrk_reduce(P, (int)d, splits, alpha, H, s) != hipSuccess) return GPTQ_ERR_HIP;
    t += n_pass;
  }
  return GPTQ_OK;
}
