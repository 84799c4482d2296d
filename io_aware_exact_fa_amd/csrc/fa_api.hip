// C ABI of libfa.so: argument validation, device check, dispatch to the
// kernel instances, no allocation, no synchronization.  The contract of every
// entry point is documented in include/fa.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "fa.h"
#include "fa_kernels.hpp"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxGridYZ = 65535;   // grid y (heads) and z (batch) limit
constexpr int kMaxDevices = 64;
constexpr int kMaxN = (1 << 23);   // keeps byte offsets inside one head matrix below 2^32
constexpr uint64_t kMaxRows = (uint64_t)1 << 34;  // keeps 1-D row grids below 2^31 blocks
constexpr uint64_t kMaxHeads = (uint64_t)1 << 24;  // B*H: with kMaxRows keeps tile grids below 2^31

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Tensor pointers: non-null and 16-byte aligned (the kernels read and write
// them in 16-byte pieces, and the LDS-direct copies move 16 bytes per lane).
template <class... P>
bool tensors_ok(P... p) {
  return ((p != nullptr && ((uintptr_t)p & 15) == 0) && ...);
}
// Float32 row statistics (lse) and int32 offsets: non-null, 4-byte aligned.
bool words_ok(const void* p) { return p != nullptr && ((uintptr_t)p & 3) == 0; }
// Rows per head of the workspace arrays: N rounded up to whole 64-row tiles.
int padded_rows(int N) { return (N + 63) / 64 * 64; }

// B*H*N*d without overflow; 0 if it does not fit comfortably in 63 bits.
uint64_t elements(int B, int H, int N, int d) {
  const unsigned __int128 n = (unsigned __int128)(uint64_t)B * (uint64_t)H * (uint64_t)N * (uint64_t)d;
  if (n > ((unsigned __int128)1 << 62)) return 0;
  return (uint64_t)n;
}

fa_status check_shape(int B, int H, int N, int d, float scale, fa_dtype dtype) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARGUMENT;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARGUMENT;
  if (elements(B, H, N, d) == 0) return FA_ERR_INVALID_ARGUMENT;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B > kMaxGridYZ || H > kMaxGridYZ) return FA_ERR_UNSUPPORTED;
  if (N > kMaxN) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)B * H * N > kMaxRows) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)B * H > kMaxHeads) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Packed variable-length batch: B sequences of at most max_s tokens, `total`
// rows per head.  The per-(sequence, head) limits are those of the dense shape
// [B, H, max_s]; in addition the packed tensors must be addressable.
fa_status check_varlen(const int* cu_seqlens, int B, int max_s, int total, int H, int H_kv, int d,
                       float scale, fa_dtype dtype) {
  if (!cu_seqlens || total <= 0) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_shape(B, H, max_s, d, scale, dtype);
  if (st != FA_OK) return st;
  if (H_kv <= 0 || H % H_kv != 0) return FA_ERR_INVALID_ARGUMENT;
  if (elements(1, H, total, d) == 0) return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

// Checks of a call description; then its grouping, packing and window into
// the kernel arguments.
fa_status check_attn(const fa_attn* p) {
  if (!p) return FA_ERR_INVALID_ARGUMENT;
  if (p->window_left < -1 || p->window_right < -1) return FA_ERR_INVALID_ARGUMENT;
  if (!(p->dropout_p >= 0.f && p->dropout_p <= 1.f)) return FA_ERR_INVALID_ARGUMENT;   // NaN too
  if (p->cu_seqlens && !words_ok(p->cu_seqlens)) return FA_ERR_INVALID_ARGUMENT;
  if (p->block_mask && p->block_mask_heads != 1 && p->block_mask_heads != p->H)
    return FA_ERR_INVALID_ARGUMENT;
  if (p->cu_seqlens)
    return check_varlen(p->cu_seqlens, p->B, p->N, p->total, p->H, p->H_kv, p->d, p->scale,
                        p->dtype);
  const fa_status st = check_shape(p->B, p->H, p->N, p->d, p->scale, p->dtype);
  if (st != FA_OK) return st;
  if (p->H_kv <= 0 || p->H % p->H_kv != 0) return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

template <class Args>
void apply_attn(const fa_attn* p, Args* a) {
  a->G = p->H / p->H_kv;
  a->cu_seqlens = p->cu_seqlens;
  a->total = p->cu_seqlens ? p->total : 0;
  // A side wider than the longest sequence is open (this also keeps i + w in range).
  a->wl = (p->window_left < 0 || p->window_left >= p->N) ? fa::kNoLimit : p->window_left;
  a->wr = (p->window_right < 0 || p->window_right >= p->N) ? fa::kNoLimit : p->window_right;
  // Keep iff the 16-bit uniform is below keep_t = round((1 - p) 2^16) (nearest, ties to even).
  const uint32_t keep_t = (uint32_t)lrint((1.0 - (double)p->dropout_p) * 65536.0);
  a->drop.keep_t = keep_t;
  a->drop.scale = keep_t > 0 ? (float)(65536.0 / keep_t) : 0.f;
  a->drop.seed_lo = (uint32_t)(p->seed & 0xFFFFFFFFu);
  a->drop.seed_hi = (uint32_t)(p->seed >> 32);
  a->drop.offset = p->rng_offset;
  if (p->block_mask) {
    a->bm.mask = p->block_mask;
    a->bm.heads = p->block_mask_heads;
    a->bm.nbq = (p->N + fa::kBlockQ - 1) / fa::kBlockQ;
    a->bm.nbk = (p->N + fa::kBlockK - 1) / fa::kBlockK;
  }
}

// 1 = gfx950, 2 = something else; 0 = not yet known.
std::atomic<int> g_device_ok[kMaxDevices];

fa_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int known = g_device_ok[dev].load(std::memory_order_relaxed);
    if (known == 1) return FA_OK;
    if (known == 2) return FA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FA_OK : FA_ERR_DEVICE;
}

// Backward workspace of fa_bwd_noalloc: one array per GPU, part of the
// library's code object, so that calls made where nothing may be allocated
// (graph capture, serving loops) still have D and L2.  The name is the host
// stand-in only; kernels get the device address that hipGetSymbolAddress
// returns for the current device, cached per device on the first call.
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of this device's `scratch`, or null if it cannot be had.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  if (dev < kMaxDevices) {
    void* known = g_scratch[dev].load(std::memory_order_acquire);
    if (known) return known;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  if (dev < kMaxDevices) g_scratch[dev].store(ptr, std::memory_order_release);
  return ptr;
}

fa::Dt to_dt(fa_dtype d) {
  return d == FA_F32 ? fa::Dt::f32 : (d == FA_F16 ? fa::Dt::f16 : fa::Dt::bf16);
}

fa_status launched(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

static_assert(FA_BLOCK_Q == fa::kBlockQ && FA_BLOCK_K == fa::kBlockK, "block sizes of fa.h");

// Bytes of the D and L2 part of the backward workspace, and of the whole
// workspace (that part, then the float32 dQ accumulator of the one-pass
// backward), for a valid shape.
size_t ws_stats_bytes(int B, int H, int N) {
  return align_up(2 * (uint64_t)B * H * padded_rows(N) * sizeof(float));
}
size_t ws_full_bytes(int B, int H, int N, int d) {
  return ws_stats_bytes(B, H, N) + align_up((uint64_t)B * H * padded_rows(N) * d * sizeof(float));
}

// Shared checks of the backward entry points, then the workspace split: the
// workspace must hold D and L2, and the whole workspace when `need_acc`; the
// accumulator is set (a->dqacc) whenever the workspace holds it.
fa_status bwd_setup(int B, int H, int H_kv, int N, int d, float scale, fa_dtype dtype,
                    void* workspace, size_t workspace_bytes, fa::BwdArgs* a,
                    bool need_acc = false);
// Sets the tensor pointers and enqueues preprocess, dK/dV and dQ.
fa_status bwd_all(fa::BwdArgs& a, const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv, int d,
                  int causal, fa_dtype dtype, void* stream);

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported dtype, head dimension or size";
    case FA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case FA_ERR_DEVICE: return "current HIP device is not a gfx950 GPU";
    case FA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

fa_status fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int H_kv, int N, int d, int causal, float scale, fa_dtype dtype,
                     void* stream) {
  if (!tensors_ok(q, k, v, o) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_shape(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (H_kv <= 0 || H % H_kv != 0) return FA_ERR_INVALID_ARGUMENT;
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, scale};
  a.G = H / H_kv;
  return launched(fa::launch_fwd(to_dt(dtype), d, causal != 0, a, (hipStream_t)stream));
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, int causal, float scale, fa_dtype dtype, void* stream) {
  return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, stream);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens, int B, int max_s, int total, int H, int H_kv,
                        int d, int causal, float scale, fa_dtype dtype, void* stream) {
  if (!tensors_ok(q, k, v, o) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens && !words_ok(cu_seqlens)) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_varlen(cu_seqlens, B, max_s, total, H, H_kv, d, scale, dtype);
  if (st != FA_OK) return st;
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, H, max_s, scale};
  a.G = H / H_kv;
  a.cu_seqlens = cu_seqlens;
  a.total = total;
  return launched(fa::launch_fwd(to_dt(dtype), d, causal != 0, a, (hipStream_t)stream));
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  if (elements(B, H, N, d) == 0) return 0;
  if (elements(B, H, padded_rows(N), d) == 0) return 0;
  return ws_stats_bytes(B, H, N);
}

fa_status fa_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H,
                            int N, int d, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!tensors_ok(o, dout) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  fa::BwdArgs a{};
  fa_status st = bwd_setup(B, H, H, N, d, 1.0f, dtype, workspace, workspace_bytes, &a);
  if (st != FA_OK) return st;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  return launched(fa::launch_bwd_pre(to_dt(dtype), d, a, (hipStream_t)stream));
}

fa_status fa_bwd_dkdv_gqa(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, void* dk, void* dv, int B, int H, int H_kv, int N,
                          int d, int causal, float scale, fa_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!tensors_ok(q, k, v, dout, dk, dv) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  fa::BwdArgs a{};
  fa_status st = bwd_setup(B, H, H_kv, N, d, scale, dtype, workspace, workspace_bytes, &a);
  if (st != FA_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dk = dk;
  a.dv = dv;
  return launched(fa::launch_bwd_dkdv(to_dt(dtype), d, causal != 0, a, (hipStream_t)stream));
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, void* dk, void* dv, int B, int H, int N, int d, int causal,
                      float scale, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return fa_bwd_dkdv_gqa(q, k, v, dout, lse, dk, dv, B, H, H, N, d, causal, scale, dtype,
                         workspace, workspace_bytes, stream);
}

fa_status fa_bwd_dq_gqa(const void* q, const void* k, const void* v, const void* dout,
                        const float* lse, void* dq, int B, int H, int H_kv, int N, int d,
                        int causal, float scale, fa_dtype dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!tensors_ok(q, k, v, dout, dq) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  fa::BwdArgs a{};
  fa_status st = bwd_setup(B, H, H_kv, N, d, scale, dtype, workspace, workspace_bytes, &a);
  if (st != FA_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  return launched(fa::launch_bwd_dq(to_dt(dtype), d, causal != 0, a, (hipStream_t)stream));
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, void* dq, int B, int H, int N, int d, int causal,
                    float scale, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return fa_bwd_dq_gqa(q, k, v, dout, lse, dq, B, H, H, N, d, causal, scale, dtype, workspace,
                       workspace_bytes, stream);
}

fa_status fa_bwd_dkdv_dq(const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, void* dk, void* dv, int B, int H, int H_kv, int N,
                         int d, int causal, float scale, fa_dtype dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!tensors_ok(q, k, v, dout, dk, dv) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;   // no one-pass instance
  fa::BwdArgs a{};
  fa_status st = bwd_setup(B, H, H_kv, N, d, scale, dtype, workspace, workspace_bytes, &a, true);
  if (st != FA_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dk = dk;
  a.dv = dv;
  return launched(fa::launch_bwd_dkdvq(to_dt(dtype), d, causal != 0, a, (hipStream_t)stream));
}

fa_status fa_bwd_dq_finalize(void* dq, int B, int H, int N, int d, float scale, fa_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!tensors_ok(dq)) return FA_ERR_INVALID_ARGUMENT;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  fa::BwdArgs a{};
  fa_status st = bwd_setup(B, H, H, N, d, scale, dtype, workspace, workspace_bytes, &a, true);
  if (st != FA_OK) return st;
  a.dq = dq;
  return launched(fa::launch_bwd_dqfin(to_dt(dtype), d, a, (hipStream_t)stream));
}

fa_status fa_fwd_ex(const fa_attn* p, const void* q, const void* k, const void* v, void* o,
                    float* lse, void* stream) {
  if (!tensors_ok(q, k, v, o) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_attn(p);
  if (st != FA_OK) return st;
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, p->B, p->H, p->N, p->scale};
  apply_attn(p, &a);
  return launched(fa::launch_fwd(to_dt(p->dtype), p->d, p->causal != 0, a, (hipStream_t)stream));
}

fa_status fa_bwd_ex(const fa_attn* p, const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!tensors_ok(q, k, v, o, dout, dq, dk, dv) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_attn(p);
  if (st != FA_OK) return st;
  fa::BwdArgs a{};
  st = bwd_setup(p->B, p->H, p->H_kv, p->N, p->d, p->scale, p->dtype, workspace, workspace_bytes,
                 &a);
  if (st != FA_OK) return st;
  apply_attn(p, &a);
  return bwd_all(a, q, k, v, o, dout, lse, dq, dk, dv, p->d, p->causal, p->dtype, stream);
}

fa_status fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv,
                     int N, int d, int causal, float scale, fa_dtype dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!tensors_ok(q, k, v, o, dout, dq, dk, dv) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  fa::BwdArgs a{};
  fa_status st = bwd_setup(B, H, H_kv, N, d, scale, dtype, workspace, workspace_bytes, &a);
  if (st != FA_OK) return st;
  return bwd_all(a, q, k, v, o, dout, lse, dq, dk, dv, d, causal, dtype, stream);
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        const int* cu_seqlens, int B, int max_s, int total, int H, int H_kv,
                        int d, int causal, float scale, fa_dtype dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!tensors_ok(q, k, v, o, dout, dq, dk, dv) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens && !words_ok(cu_seqlens)) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_varlen(cu_seqlens, B, max_s, total, H, H_kv, d, scale, dtype);
  if (st != FA_OK) return st;
  fa::BwdArgs a{};
  st = bwd_setup(B, H, H_kv, max_s, d, scale, dtype, workspace, workspace_bytes, &a);
  if (st != FA_OK) return st;
  a.cu_seqlens = cu_seqlens;
  a.total = total;
  return bwd_all(a, q, k, v, o, dout, lse, dq, dk, dv, d, causal, dtype, stream);
}


fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                 int causal, float scale, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream);
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int H, int N, int d, int causal, float scale, fa_dtype dtype,
                         void* stream) {
  if (!tensors_ok(q, k, v, o, dout, dq, dk, dv) || !words_ok(lse)) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_shape(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (ws_stats_bytes(B, H, N) > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  st = check_device();
  if (st != FA_OK) return st;
  void* ws = scratch_address();
  if (!ws) return FA_ERR_DEVICE;
  fa::BwdArgs a{};
  // D and L2 only: the two-pass backward (dQ by its own pass, no accumulator).
  st = bwd_setup(B, H, H, N, d, scale, dtype, ws, ws_stats_bytes(B, H, N), &a);
  if (st != FA_OK) return st;
  return bwd_all(a, q, k, v, o, dout, lse, dq, dk, dv, d, causal, dtype, stream);
}

}  // extern "C"

namespace {

fa_status bwd_setup(int B, int H, int H_kv, int N, int d, float scale, fa_dtype dtype,
                    void* workspace, size_t workspace_bytes, fa::BwdArgs* a, bool need_acc) {
  fa_status st = check_shape(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (H_kv <= 0 || H % H_kv != 0) return FA_ERR_INVALID_ARGUMENT;
  const size_t stats = ws_stats_bytes(B, H, N), full = ws_full_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < (need_acc ? full : stats) ||
      ((uintptr_t)workspace % kAlign) != 0)
    return FA_ERR_WORKSPACE;
  st = check_device();
  if (st != FA_OK) return st;
  a->Np = padded_rows(N);
  a->delta = static_cast<float*>(workspace);
  a->l2 = a->delta + (size_t)B * H * a->Np;
  a->dqacc = workspace_bytes >= full
                 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + stats)
                 : nullptr;
  a->B = B;
  a->H = H;
  a->N = N;
  a->scale = scale;
  a->G = H / H_kv;
  return FA_OK;
}

fa_status bwd_all(fa::BwdArgs& a, const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv, int d,
                  int causal, fa_dtype dtype, void* stream) {
  fa_status st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const fa::Dt dt = to_dt(dtype);
  hipStream_t s = (hipStream_t)stream;
  // The two-pass backward (dQ by its own pass; no accumulator to zero, even
  // when the caller's workspace could hold one).
  a.dqacc = nullptr;
  st = launched(fa::launch_bwd_pre(dt, d, a, s));
  if (st != FA_OK) return st;
  st = launched(fa::launch_bwd_dkdv(dt, d, causal != 0, a, s));
  if (st != FA_OK) return st;
  return launched(fa::launch_bwd_dq(dt, d, causal != 0, a, s));
}

}  // namespace
