// The no-allocation variant of decode attention: the same kernels as
// spa_decode_attn, with their scratch (the softmax partials of the pieces
// and the device error word) in a fixed array of the library instead of a
// caller workspace, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array; every GPU the library runs on
// holds its own copy until the process ends. In host code its name is only
// a host-side stand-in, so its device address is looked up once per device
// (hipGetSymbolAddress, with that device current, from spa_init) and that
// address - never the name - is what kernels and fills receive.
#include <mutex>
#include <string>

#include "host.h"

namespace {

constexpr size_t kScratchErrBytes = 256;                    // the error word (and padding)
constexpr size_t kScratchPartBytes = (size_t)24 << 20;      // piece partials: 24 MiB
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchErrBytes + kScratchPartBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

namespace spa {

spa_status noalloc_bind_device(int device) {
  if (device < 0 || device >= kMaxDevices) return fail(SPA_EUNSUPPORTED, "device index above the scratch table");
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[device]) return SPA_OK;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
  }
  g_scratch[device] = p;
  return SPA_OK;
}

}  // namespace spa

using namespace spa;

extern "C" spa_status spa_decode_attn_noalloc(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l,
                                              const spa_batch* b, int32_t tok0, int32_t n_tok, const void* q,
                                              void* o_out, int32_t* err_out, void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = check_decode_attn_args(m, l, b, tok0, n_tok, q, o_out);
  if (rc) return rc;
  if (((uintptr_t)err_out) & 3) return fail(SPA_EINVAL, "err_out must be 4-byte aligned");
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    base = ctx->device >= 0 && ctx->device < kMaxDevices ? g_scratch[ctx->device] : nullptr;
  }
  if (!base) return fail(SPA_EHIP, "no scratch address for this device (spa_init did not bind it)");
  unsigned char* sb = static_cast<unsigned char*>(base);
  int32_t* err_word = err_out ? err_out : reinterpret_cast<int32_t*>(sb);
  float* part = reinterpret_cast<float*>(sb + kScratchErrBytes);
  return decode_attn_on_scratch(ctx, m, l, b, tok0, n_tok, q, o_out, part, kScratchPartBytes, err_word,
                                err_out == nullptr, (hipStream_t)stream);
}
