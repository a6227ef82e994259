// C-ABI layer: argument validation, workspace sizing and dispatch to the kernels.
// Declared in include/fa.h. Every check happens on the host before any HIP call, so an
// invalid request launches nothing and writes nothing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

thread_local char g_last_error[256] = "";
thread_local fa::KernelTimer g_timer;

// Hands out (and clears) the pending measurement events of this thread. The launch code
// records them as it goes (KernelTimer::mark), so each call gets its own copy.
fa::KernelTimer take_timer() {
  fa::KernelTimer t = g_timer;
  g_timer = fa::KernelTimer{};
  return t;
}

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shared validation of the sizes and the tensor pointers.
fa_status check_common(fa_dtype dt, int B, int H, int N, int d, float scale) {
  if (dt != FA_F32 && dt != FA_BF16) return fail(FA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
    return fail(FA_ERR_INVALID, "sizes must be positive (B=%d H=%d N=%d d=%d)", B, H, N, d);
  const long double elems = (long double)B * H * N * d;
  if (elems * 4 > (long double)(1ull << 62)) return fail(FA_ERR_INVALID, "tensor size overflows");
  const long long wgs = (long long)B * H * ((N + fa::kFwdRowsPerWG - 1) / fa::kFwdRowsPerWG);
  if (wgs > 0x7fffffffLL) return fail(FA_ERR_INVALID, "grid too large (B*H*ceil(N/128) > 2^31-1)");
  if (N > fa::kMaxSeqLen) return fail(FA_ERR_UNSUPPORTED, "N=%d beyond the supported %d", N, fa::kMaxSeqLen);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite");
  if (d != 16 && d != 32 && d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension %d not built (16, 32, 64, 128)", d);
  return FA_OK;
}

fa_status check_tensor(const void* p, const char* name, size_t align) {
  if (p == nullptr) return fail(FA_ERR_INVALID, "%s is NULL", name);
  if (!aligned(p, align)) return fail(FA_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
  return FA_OK;
}

#define FA_TRY(expr)                 \
  do {                               \
    fa_status _s = (expr);           \
    if (_s != FA_OK) return _s;      \
  } while (0)

fa_status check_mask(const uint8_t* mask, int mask_block, int N, int tile_keys) {
  if (mask == nullptr) return fail(FA_ERR_INVALID, "block_mask is NULL");
  if (mask_block <= 0 || mask_block % fa::kFwdRowsPerWG != 0)
    return fail(FA_ERR_INVALID, "mask_block must be a positive multiple of 128 (got %d)", mask_block);
  if ((N + tile_keys - 1) / tile_keys > fa::kMaxTileList)
    return fail(FA_ERR_UNSUPPORTED, "block-sparse path supports at most %d key tiles (N=%d)",
                fa::kMaxTileList, N);
  return FA_OK;
}

// Dropout parameters: threshold floor(p 2^16) on a 16-bit generator value, scale 1 / (1 - p).
struct DropoutParams {
  bool on = false;
  uint32_t thr = 0, seed_lo = 0, seed_hi = 0;
  float scale = 1.0f;
};

fa_status make_dropout(float p, uint64_t seed, DropoutParams* out) {
  if (!(p >= 0.0f && p < 1.0f)) return fail(FA_ERR_INVALID, "dropout_p must be in [0, 1) (got %g)", (double)p);
  DropoutParams d;
  d.on = p > 0.0f;
  d.thr = (uint32_t)std::min(std::floor((double)p * 65536.0), 65535.0);
  d.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  d.seed_hi = (uint32_t)(seed >> 32);
  d.scale = (float)(1.0 / (1.0 - (double)p));
  *out = d;
  return FA_OK;
}

fa_status fwd_impl(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k,
                   const void* v, void* o, float* lse, float scale, int causal,
                   const int32_t* kv_len, const uint8_t* mask, int mask_block, bool sparse,
                   hipStream_t stream, const DropoutParams& drop = DropoutParams{}) {
  FA_TRY(check_common(dt, B, H, N, d, scale));
  if (dt == FA_F32 && d == 16) return fail(FA_ERR_UNSUPPORTED, "fp32 forward is built for d in {32, 64, 128}");
  FA_TRY(check_tensor(q, "q", 16));
  FA_TRY(check_tensor(k, "k", 16));
  FA_TRY(check_tensor(v, "v", 16));
  FA_TRY(check_tensor(o, "o", 16));
  FA_TRY(check_tensor(lse, "lse", 4));
  if (kv_len && !aligned(kv_len, 4)) return fail(FA_ERR_INVALID, "kv_len is not 4-byte aligned");
  if (sparse)
    FA_TRY(check_mask(mask, mask_block, N, dt == FA_BF16 ? fa::fwd_tile_keys_bf16(d) : fa::kFwdTileKeysF32));

  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.kv_len = kv_len;
  a.mask = sparse ? mask : nullptr;
  a.B = B;
  a.H = H;
  a.N = N;
  a.mb = sparse ? mask_block : 0;
  a.nb = sparse ? (N + mask_block - 1) / mask_block : 0;
  const int rows_per_wg = dt == FA_BF16 ? fa::kFwdRowsPerWGBF16 : fa::kFwdRowsPerWG;
  a.ntq = (N + rows_per_wg - 1) / rows_per_wg;
  a.causal = causal ? 1 : 0;
  const float sabs = std::fabs(scale);
  // The online maximum needs a positive exponent scale. A negative scale is applied by
  // negating Q (exact); a zero scale by zeroing Q (every allowed score is then 0).
  a.qmul = scale > 0.f ? 1.f : (scale < 0.f ? -1.f : 0.f);
  a.c2 = scale != 0.f ? sabs * 1.4426950408889634f : 1.4426950408889634f;
  a.sc_abs = sabs;
  a.wl = -1;
  a.wr = causal ? 0 : -1;
  a.cu = nullptr;
  a.rs = d;
  a.total = 0;
  a.drop_thr = drop.thr;
  a.seed_lo = drop.seed_lo;
  a.seed_hi = drop.seed_hi;
  a.drop_scale = drop.scale;
  fa::KernelTimer tm = take_timer();
  hipError_t e = fa::launch_fwd(a, dt, d, stream, tm, drop.on);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

// A window extent that reaches past every position of a sequence of at most max_seqlen
// tokens (i - j and j - i never exceed max_seqlen - 1) allows every key: it is replaced by
// -1 (unbounded), so the kernels never add an extent near INT_MAX to a row index.
int clamp_window(int extent, int max_seqlen) { return extent >= max_seqlen ? -1 : extent; }

// Shared validation of the packed variable-length calls.
fa_status check_varlen(fa_dtype dt, int nseq, int H, int total, int max_seqlen, int d, float scale,
                       const int32_t* cu, int window_left, int window_right) {
  if (dt != FA_F32 && dt != FA_BF16) return fail(FA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (nseq <= 0 || H <= 0 || total < 0 || max_seqlen < 0 || d <= 0)
    return fail(FA_ERR_INVALID, "sizes must be positive (nseq=%d H=%d total=%d max_seqlen=%d d=%d)", nseq, H,
                total, max_seqlen, d);
  if ((long double)total * H * d * 4 > (long double)(1ull << 62)) return fail(FA_ERR_INVALID, "tensor size overflows");
  const long long wgs = (long long)nseq * H * ((max_seqlen + fa::kFwdRowsPerWG - 1) / fa::kFwdRowsPerWG);
  if (wgs > 0x7fffffffLL) return fail(FA_ERR_INVALID, "grid too large (nseq*H*ceil(max_seqlen/128) > 2^31-1)");
  if (max_seqlen > fa::kMaxSeqLen)
    return fail(FA_ERR_UNSUPPORTED, "max_seqlen %d beyond the supported %d", max_seqlen, fa::kMaxSeqLen);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite");
  if (cu == nullptr) return fail(FA_ERR_INVALID, "cu_seqlens is NULL");
  if (!aligned(cu, 4)) return fail(FA_ERR_INVALID, "cu_seqlens is not 4-byte aligned");
  if (window_left < -1 || window_right < -1)
    return fail(FA_ERR_INVALID, "window extents must be >= 0, or -1 for unbounded");
  if (dt != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "packed sequences are built for bf16 only");
  if (d != 16 && d != 32 && d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension %d not built (16, 32, 64, 128)", d);
  return FA_OK;
}

// Workspace layout of the key/value-cache forward: part_u, part_m, part_l (each 256-byte
// aligned). Returns 0 for invalid sizes.
size_t kvcache_ws(int B, int H, int Nq, int Nk, int d, size_t* off_m, size_t* off_l) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
  if ((long double)B * H * (long double)(Nq > Nk ? Nq : Nk) * d * 4 > (long double)(1ull << 62)) return 0;
  const size_t slots = (size_t)fa::kvcache_max_waves(B, H, Nk) + (size_t)B * H - 1;
  const size_t rows = slots * Nq;
  const size_t su = align256(rows * d * sizeof(float)), sm = align256(rows * sizeof(float));
  if (off_m) *off_m = su;
  if (off_l) *off_l = su + sm;
  return su + 2 * sm;
}

}  // namespace

extern "C" {

fa_status fa_fwd(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k,
                 const void* v, void* o, float* lse, float scale, int causal,
                 const int32_t* kv_len, hipStream_t stream) {
  return fwd_impl(dt, B, H, N, d, q, k, v, o, lse, scale, causal, kv_len, nullptr, 0, false, stream);
}

fa_status fa_fwd_blocksparse(fa_dtype dt, int B, int H, int N, int d, const void* q,
                             const void* k, const void* v, void* o, float* lse, float scale,
                             int causal, const int32_t* kv_len, const uint8_t* block_mask,
                             int mask_block, hipStream_t stream) {
  return fwd_impl(dt, B, H, N, d, q, k, v, o, lse, scale, causal, kv_len, block_mask, mask_block,
                  true, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  const long double rows = (long double)B * H * N;
  if (rows * d * 4 > (long double)(1ull << 62)) return 0;
  return align256((size_t)B * H * N * sizeof(float)) + fa::kMaxKeyTiles * sizeof(uint32_t);
}

}  // extern "C"

namespace {

fa_status bwd_impl(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k,
                   const void* v, const void* o, const void* dout, const float* lse, void* dq,
                   void* dk, void* dv, float scale, int causal, const int32_t* kv_len,
                   const uint8_t* block_mask, int mask_block, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, const DropoutParams& drop) {
  FA_TRY(check_common(dt, B, H, N, d, scale));
  if (dt != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "backward is built for bf16 only");
  FA_TRY(check_tensor(q, "q", 16));
  FA_TRY(check_tensor(k, "k", 16));
  FA_TRY(check_tensor(v, "v", 16));
  FA_TRY(check_tensor(o, "o", 16));
  FA_TRY(check_tensor(dout, "dout", 16));
  FA_TRY(check_tensor(lse, "lse", 4));
  FA_TRY(check_tensor(dq, "dq", 16));
  FA_TRY(check_tensor(dk, "dk", 16));
  FA_TRY(check_tensor(dv, "dv", 16));
  if (kv_len && !aligned(kv_len, 4)) return fail(FA_ERR_INVALID, "kv_len is not 4-byte aligned");
  if (block_mask) FA_TRY(check_mask(block_mask, mask_block, N, fa::kBwdMinTile));
  const size_t need = fa_bwd_workspace_bytes(B, H, N, d);
  if (workspace == nullptr) return fail(FA_ERR_INVALID, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);

  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsum = reinterpret_cast<float*>(workspace);
  a.order = block_mask ? reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(workspace) +
                                                     align256((size_t)B * H * N * sizeof(float)))
                       : nullptr;
  a.kv_len = kv_len;
  a.mask = block_mask;
  a.B = B;
  a.H = H;
  a.N = N;
  a.mb = block_mask ? mask_block : 0;
  a.nb = block_mask ? (N + mask_block - 1) / mask_block : 0;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  a.c2s = scale * 1.4426950408889634f;
  a.wl = -1;
  a.wr = causal ? 0 : -1;
  a.cu = nullptr;
  a.rs = d;
  a.total = 0;
  a.drop_thr = drop.thr;
  a.seed_lo = drop.seed_lo;
  a.seed_hi = drop.seed_hi;
  a.drop_scale = drop.scale;
  a.dropout = drop.on ? 1 : 0;
  fa::KernelTimer tm = take_timer();
  hipError_t e = fa::launch_bwd(a, d, stream, tm);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_bwd(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k,
                 const void* v, const void* o, const void* dout, const float* lse, void* dq,
                 void* dk, void* dv, float scale, int causal, const int32_t* kv_len,
                 const uint8_t* block_mask, int mask_block, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(dt, B, H, N, d, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, kv_len, block_mask,
                  mask_block, workspace, workspace_bytes, stream, DropoutParams{});
}

fa_status fa_fwd_dropout(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k,
                         const void* v, void* o, float* lse, float scale, int causal,
                         const int32_t* kv_len, float dropout_p, uint64_t seed, hipStream_t stream) {
  DropoutParams drop;
  FA_TRY(make_dropout(dropout_p, seed, &drop));
  if (drop.on && dt != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "dropout is built for bf16 only");
  return fwd_impl(dt, B, H, N, d, q, k, v, o, lse, scale, causal, kv_len, nullptr, 0, false, stream, drop);
}

fa_status fa_bwd_dropout(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k,
                         const void* v, const void* o, const void* dout, const float* lse, void* dq,
                         void* dk, void* dv, float scale, int causal, const int32_t* kv_len,
                         float dropout_p, uint64_t seed, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  DropoutParams drop;
  FA_TRY(make_dropout(dropout_p, seed, &drop));
  return bwd_impl(dt, B, H, N, d, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, kv_len, nullptr, 0,
                  workspace, workspace_bytes, stream, drop);
}

size_t fa_fwd_kvcache_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  return kvcache_ws(B, H, Nq, Nk, d, nullptr, nullptr);
}

}  // extern "C"

namespace {

// Device scratch of fa_fwd_kvcache_noalloc: the key split's partial results live here
// instead of in a caller workspace. Each device that runs the call holds its own copy
// until the process ends. In host code `scratch` only names the symbol; the device
// address comes from hipGetSymbolAddress, looked up once per device (scratch_ptr).
constexpr size_t kNoAllocScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (nullptr with *status set on failure).
void* scratch_ptr(fa_status* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(FA_ERR_UNSUPPORTED, "device %d beyond the %d devices the scratch table covers", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *status = fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Shared body of the two cache-forward calls. With use_scratch the partial results go to
// the current device's static scratch (workspace and workspace_bytes are ignored).
fa_status kvcache_impl(fa_dtype dt, int B, int H, int Nq, int Nk, int d, const void* q, const void* k_cache,
                       const void* v_cache, void* o, float* lse, float scale, int causal, const int32_t* kv_len,
                       void* workspace, size_t workspace_bytes, bool use_scratch, hipStream_t stream) {
  if (dt != FA_F32 && dt != FA_BF16) return fail(FA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0)
    return fail(FA_ERR_INVALID, "sizes must be positive (B=%d H=%d Nq=%d Nk=%d d=%d)", B, H, Nq, Nk, d);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite");
  size_t off_m = 0, off_l = 0;
  const size_t need = kvcache_ws(B, H, Nq, Nk, d, &off_m, &off_l);
  if (need == 0) return fail(FA_ERR_INVALID, "tensor size overflows");
  if (dt != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "key/value-cache forward is built for bf16 only");
  if (d != 16 && d != 32 && d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension %d not built (16, 32, 64, 128)", d);
  if (Nq > fa::kDecMaxQueries)
    return fail(FA_ERR_UNSUPPORTED, "at most %d queries per (b, h) (got Nq=%d)", fa::kDecMaxQueries, Nq);
  FA_TRY(check_tensor(q, "q", 16));
  FA_TRY(check_tensor(k_cache, "k_cache", 16));
  FA_TRY(check_tensor(v_cache, "v_cache", 16));
  FA_TRY(check_tensor(o, "o", 16));
  FA_TRY(check_tensor(lse, "lse", 4));
  if (kv_len && !aligned(kv_len, 4)) return fail(FA_ERR_INVALID, "kv_len is not 4-byte aligned");
  if (use_scratch) {
    if (need > kNoAllocScratchBytes)
      return fail(FA_ERR_UNSUPPORTED, "partial results need %zu bytes, beyond the %zu-byte static scratch", need,
                  kNoAllocScratchBytes);
  } else {
    if (workspace == nullptr) return fail(FA_ERR_INVALID, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  }

  fa::DecArgs a{};
  if ((long long)B * H * ((Nk + 31) / 32) > 0x7fffffffLL || (long long)B * H + fa::kDecMaxWaves > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "cache too large (B*H*ceil(Nk/32) key tiles or B*H + %d partial-result "
                "slots beyond 2^31-1)", fa::kDecMaxWaves);
  if ((long long)B * H * Nq > 0x7fffffffLL) return fail(FA_ERR_INVALID, "grid too large (B*H*Nq > 2^31-1)");
  if (use_scratch) {
    fa_status st = FA_OK;
    workspace = scratch_ptr(&st);
    if (workspace == nullptr) return st;
  }
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.lse = lse;
  a.kv_len = kv_len;
  char* ws = reinterpret_cast<char*>(workspace);
  a.part_u = reinterpret_cast<float*>(ws);
  a.part_m = reinterpret_cast<float*>(ws + off_m);
  a.part_l = reinterpret_cast<float*>(ws + off_l);
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.causal = causal ? 1 : 0;
  const float sabs = std::fabs(scale);
  a.qmul = scale > 0.f ? 1.f : (scale < 0.f ? -1.f : 0.f);
  a.c2 = scale != 0.f ? sabs * 1.4426950408889634f : 1.4426950408889634f;
  a.sc_abs = sabs;
  fa::KernelTimer tm = take_timer();
  hipError_t e = fa::launch_kvcache(a, d, stream, tm);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "key/value-cache forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd_kvcache(fa_dtype dt, int B, int H, int Nq, int Nk, int d, const void* q,
                         const void* k_cache, const void* v_cache, void* o, float* lse,
                         float scale, int causal, const int32_t* kv_len, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return kvcache_impl(dt, B, H, Nq, Nk, d, q, k_cache, v_cache, o, lse, scale, causal, kv_len, workspace,
                      workspace_bytes, false, stream);
}

fa_status fa_fwd_kvcache_noalloc(fa_dtype dt, int B, int H, int Nq, int Nk, int d, const void* q,
                                 const void* k_cache, const void* v_cache, void* o, float* lse, float scale,
                                 int causal, const int32_t* kv_len, hipStream_t stream) {
  return kvcache_impl(dt, B, H, Nq, Nk, d, q, k_cache, v_cache, o, lse, scale, causal, kv_len, nullptr, 0, true,
                      stream);
}

fa_status fa_fwd_varlen(fa_dtype dt, int nseq, int H, int total, int max_seqlen, int d,
                        const int32_t* cu_seqlens, const void* q, const void* k, const void* v, void* o,
                        float* lse, float scale, int causal, int window_left, int window_right,
                        hipStream_t stream) {
  FA_TRY(check_varlen(dt, nseq, H, total, max_seqlen, d, scale, cu_seqlens, window_left, window_right));
  if (total == 0 || max_seqlen == 0) return FA_OK;  // no token: nothing to compute
  FA_TRY(check_tensor(q, "q", 16));
  FA_TRY(check_tensor(k, "k", 16));
  FA_TRY(check_tensor(v, "v", 16));
  FA_TRY(check_tensor(o, "o", 16));
  FA_TRY(check_tensor(lse, "lse", 4));
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = nseq;
  a.H = H;
  a.N = max_seqlen;
  a.ntq = (max_seqlen + fa::kFwdRowsPerWGBF16 - 1) / fa::kFwdRowsPerWGBF16;
  a.causal = causal ? 1 : 0;
  const float sabs = std::fabs(scale);
  a.qmul = scale > 0.f ? 1.f : (scale < 0.f ? -1.f : 0.f);
  a.c2 = scale != 0.f ? sabs * 1.4426950408889634f : 1.4426950408889634f;
  a.sc_abs = sabs;
  a.wl = clamp_window(window_left, max_seqlen);
  a.wr = causal ? 0 : clamp_window(window_right, max_seqlen);
  a.cu = cu_seqlens;
  a.rs = H * d;
  a.total = total;
  fa::KernelTimer tm = take_timer();
  hipError_t e = fa::launch_fwd(a, dt, d, stream, tm);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

size_t fa_bwd_varlen_workspace_bytes(int H, int total, int d) {
  if (H <= 0 || total < 0 || d <= 0) return 0;
  if ((long double)total * H * d * 4 > (long double)(1ull << 62)) return 0;
  return align256((size_t)total * H * sizeof(float));
}

fa_status fa_bwd_varlen(fa_dtype dt, int nseq, int H, int total, int max_seqlen, int d,
                        const int32_t* cu_seqlens, const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float scale, int causal, int window_left, int window_right, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  FA_TRY(check_varlen(dt, nseq, H, total, max_seqlen, d, scale, cu_seqlens, window_left, window_right));
  if (total == 0 || max_seqlen == 0) return FA_OK;
  FA_TRY(check_tensor(q, "q", 16));
  FA_TRY(check_tensor(k, "k", 16));
  FA_TRY(check_tensor(v, "v", 16));
  FA_TRY(check_tensor(o, "o", 16));
  FA_TRY(check_tensor(dout, "dout", 16));
  FA_TRY(check_tensor(lse, "lse", 4));
  FA_TRY(check_tensor(dq, "dq", 16));
  FA_TRY(check_tensor(dk, "dk", 16));
  FA_TRY(check_tensor(dv, "dv", 16));
  const size_t need = fa_bwd_varlen_workspace_bytes(H, total, d);
  if (workspace == nullptr) return fail(FA_ERR_INVALID, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsum = reinterpret_cast<float*>(workspace);
  a.order = nullptr;
  a.kv_len = nullptr;
  a.mask = nullptr;
  a.B = nseq;
  a.H = H;
  a.N = max_seqlen;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  a.c2s = scale * 1.4426950408889634f;
  a.wl = clamp_window(window_left, max_seqlen);
  a.wr = causal ? 0 : clamp_window(window_right, max_seqlen);
  a.cu = cu_seqlens;
  a.rs = H * d;
  a.total = total;
  a.dropout = 0;
  fa::KernelTimer tm = take_timer();
  hipError_t e = fa::launch_bwd(a, d, stream, tm);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

void fa_time_next_call(const hipEvent_t* events, int n) {
  g_timer = fa::KernelTimer{};
  if (events == nullptr || n <= 0) return;
  const int m = std::min(n, fa::KernelTimer::kMax);
  for (int i = 0; i < m; ++i) {
    if (events[i] == nullptr) return;  // an incomplete list clears the request
    g_timer.ev[i] = events[i];
  }
  g_timer.n = m;
}

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID: return "FA_ERR_INVALID: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: request not implemented by this build";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
  }
  return "unknown fa_status";
}

const char* fa_last_error(void) { return g_last_error; }

}  // extern "C"
