// Forward kernels: tiled exact attention with online softmax (gfx950).
//
// Method: aiwiki.page "FlashAttention", section "Tiling and online normalization" — per
// query row keep a running maximum m, a running sum l of exp(s - m) and an accumulator u
// of exp(s - m) v; when a new key tile raises the maximum, rescale l and u by exp(m - m');
// at the end O = u / l. sendsoonai.com "FlashAttention: IO-aware explained", section
// "Tiling and exact softmax": one query block stays on chip while key/value blocks stream
// past, so the N x N score matrix never reaches HBM. Only lse = m + ln l is written.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows, 32 per wave):
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows are
//     the A operand (16-byte LDS reads), the wave's Q rows the B operand (registers, loaded
//     once). In the accumulator each lane then owns ONE query (l % 32) and 16 keys per
//     32-key block, so the row max / row sum are in-lane reductions plus one exchange
//     between the two half-waves.
//   * The unnormalised output is accumulated transposed too, O^T += V^T P^T: the
//     probabilities are used straight from the score accumulator as the B operand, and
//     V^T comes from the row-major V tile through ds_read_b64_tr_b16 transpose reads.
//   * K and V tiles (64 keys) are double-buffered in LDS; the next tile's global loads are
//     in flight while the current tile is computed.
//   * The running maximum is refreshed lazily: the accumulator is rescaled only when some
//     row's maximum grew by more than 2^8 in the exp2 domain, which keeps every
//     probability below 256 and leaves the result exact up to rounding (u and l always
//     share the same reference maximum).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBR = 128;  // query rows per workgroup
constexpr int kBC = 64;   // keys per tile
constexpr int kThreads = 256;
constexpr int kMaxTiles = 4096;  // key-tile list capacity (block-sparse)
constexpr float kRescaleLog2 = 8.0f;

// Builds, in LDS, the list of key tiles [0, ntk) whose mask block is nonzero for mask row
// `rb`. Returns the count (uniform across the workgroup).
__device__ int build_tile_list(uint16_t* list, int* wcount, const uint8_t* mask, int rb, int nb,
                               int mb, int ntk, int bc) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  int count = 0;
  for (int base = 0; base < ntk; base += kThreads) {
    const int j = base + tid;
    const bool keep = j < ntk && mask[(size_t)rb * nb + (j * bc) / mb] != 0;
    const uint64_t bal = __ballot(keep);
    const int pre = __popcll(bal & ((1ull << l) - 1ull));
    if (l == 0) wcount[w] = __popcll(bal);
    __syncthreads();
    int off = count;
    for (int i = 0; i < w; ++i) off += wcount[i];
    if (keep) list[off + pre] = (uint16_t)j;
    count += wcount[0] + wcount[1] + wcount[2] + wcount[3];
    __syncthreads();
  }
  return count;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int NCH = kBC * CH / kThreads;     // chunks per thread per tensor
  constexpr int TILE = kBC * D * 2;            // bytes of one K or V tile
  constexpr int KS = D / 16;                   // k-steps of the score product
  constexpr int MD = D / 32;                   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE];
  __shared__ uint16_t tlist[kMaxTiles];
  __shared__ int wcount[4];

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qt = a.ntq - 1 - blockIdx.x / BH;  // longest (causal) tiles first
  const int b = bh / a.H;
  const int q0 = qt * kBR;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, ql = l & 31;
  const int qi = q0 + 32 * w + ql;
  const size_t hoff = (size_t)bh * a.N * D;
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q) + hoff;
  const __bf16* __restrict__ K = reinterpret_cast<const __bf16*>(a.k) + hoff;
  const __bf16* __restrict__ V = reinterpret_cast<const __bf16*>(a.v) + hoff;

  int kv_end = a.N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), a.N);
  int hi = kv_end;
  if (a.causal) hi = min(hi, q0 + kBR);
  const int ntk = (hi + kBC - 1) / kBC;
  int ntiles = ntk;
  if (a.mask) ntiles = build_tile_list(tlist, wcount, a.mask, q0 / a.mb, a.nb, a.mb, ntk, kBC);

  // Q fragments: B operand of S^T = K Q^T, lane holds Q[qi][16 ks + 8h .. +7].
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qi < a.N) {
      qf[ks] = __builtin_bit_cast(bf16x8, gload16(Q + (size_t)qi * D + 16 * ks + 8 * h));
      if (a.qmul != 1.0f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)qf[ks][e] * a.qmul);
      }
    } else {
      qf[ks] = bf16x8{};
    }
  }

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;

  u32x4 kr[NCH], vr[NCH];
  auto gload_tile = [&](int jt) {
    const int key0 = jt * kBC;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int id = tid + kThreads * c;
      const int row = id / CH, col = (id % CH) * 8;
      const int key = key0 + row;
      if (key < a.N) {
        kr[c] = gload16(K + (size_t)key * D + col);
        vr[c] = gload16(V + (size_t)key * D + col);
      } else {
        kr[c] = u32x4{};
        vr[c] = u32x4{};
      }
    }
  };
  auto lds_store_tile = [&](int buf) {
    FA_LDS char* kb = (FA_LDS char*)smem + buf * 2 * TILE;
    FA_LDS char* vb = kb + TILE;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int id = tid + kThreads * c;
      const int row = id / CH, col = (id % CH) * 8;
      lds_store16(kb + tile_off<D>(row, col), kr[c]);
      lds_store16(vb + tile_off<D>(row, col), vr[c]);
    }
  };

  if (ntiles > 0) {
    gload_tile(a.mask ? tlist[0] : 0);
    lds_store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int jt = a.mask ? tlist[t] : t;
    const int buf = t & 1;
    if (t + 1 < ntiles) gload_tile(a.mask ? tlist[t + 1] : t + 1);

    const int key0 = jt * kBC;
    // A wave whose queries all precede the tile (causal) has nothing to do here.
    const bool active = !(a.causal && key0 > q0 + 32 * w + 31);
    if (active) {
      const FA_LDS char* kb = (const FA_LDS char*)smem + buf * 2 * TILE;
      const FA_LDS char* vb = kb + TILE;
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[mb] = mfma32(lds_read8<D>(kb, 32 * mb + ql, 16 * ks + 8 * h), qf[ks], s[mb]);
      }
      const bool edge = (key0 + kBC > kv_end) || (a.causal && key0 + kBC - 1 > q0 + 32 * w);
      if (edge) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key >= kv_end || (a.causal && key > qi)) s[mb][i] = kNegInf;
          }
      }
      float tmax = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mb][i]);
      tmax = fmaxf(tmax, wave_xor32(tmax));
      const float mcand = fmaxf(m_run, tmax);
      const bool need = (mcand - m_run) * c2 > kRescaleLog2;
      if (__ballot(need)) {
        const float alpha = need ? fast_exp2((m_run - mcand) * c2) : 1.0f;
        if (need) m_run = mcand;
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md] *= alpha;
      }
      const float moff = (m_run == kNegInf) ? 0.f : m_run * c2;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[mb][i], c2, -moff));
          s[mb][i] = p;
          l_run += p;
        }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 bp = pack8(s[st >> 1], 8 * (st & 1));
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md] = mfma32(lds_read_tr8<D>(vb, 16 * st, 32 * md), bp, o[md]);
      }
    }
    if (t + 1 < ntiles) lds_store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + wave_xor32(l_run);
  if (qi < a.N) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    __bf16* O = reinterpret_cast<__bf16*>(a.o) + hoff + (size_t)qi * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(o[md][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(O + 32 * md + 8 * g + 4 * h) = ov;
      }
    if (h == 0) a.lse[(size_t)bh * a.N + qi] = l_tot > 0.f ? m_run * a.sc_abs + logf(l_tot) : kNegInf;
  }
}

// fp32 forward: same structure on v_mfma_f32_32x32x2_f32, 32-key tiles, one LDS buffer.
template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BC = 32;
  constexpr int LD = D + 1;  // padded row stride (floats)
  constexpr int MD = D / 32;
  __shared__ float kt[BC * LD];
  __shared__ float vt[BC * LD];
  __shared__ uint16_t tlist[kMaxTiles];
  __shared__ int wcount[4];

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qt = a.ntq - 1 - blockIdx.x / BH;
  const int b = bh / a.H;
  const int q0 = qt * kBR;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, ql = l & 31;
  const int qi = q0 + 32 * w + ql;
  const size_t hoff = (size_t)bh * a.N * D;
  const float* __restrict__ Q = reinterpret_cast<const float*>(a.q) + hoff;
  const float* __restrict__ K = reinterpret_cast<const float*>(a.k) + hoff;
  const float* __restrict__ V = reinterpret_cast<const float*>(a.v) + hoff;

  int kv_end = a.N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), a.N);
  int hi = kv_end;
  if (a.causal) hi = min(hi, q0 + kBR);
  const int ntk = (hi + BC - 1) / BC;
  int ntiles = ntk;
  if (a.mask) ntiles = build_tile_list(tlist, wcount, a.mask, q0 / a.mb, a.nb, a.mb, ntk, BC);

  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = qi < a.N ? Q[(size_t)qi * D + 2 * s + h] * a.qmul : 0.f;

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;

  for (int t = 0; t < ntiles; ++t) {
    const int jt = a.mask ? tlist[t] : t;
    const int key0 = jt * BC;
    for (int e = tid; e < BC * D; e += kThreads) {
      const int row = e / D, col = e % D;
      const int key = key0 + row;
      kt[row * LD + col] = key < a.N ? K[(size_t)key * D + col] : 0.f;
      vt[row * LD + col] = key < a.N ? V[(size_t)key * D + col] : 0.f;
    }
    __syncthreads();
    if (!(a.causal && key0 > q0 + 32 * w + 31)) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 2; ++st) s = mfma32_f32(kt[ql * LD + 2 * st + h], qf[st], s);
      float tmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key >= kv_end || (a.causal && key > qi)) s[i] = kNegInf;
        tmax = fmaxf(tmax, s[i]);
      }
      tmax = fmaxf(tmax, wave_xor32(tmax));
      const float mcand = fmaxf(m_run, tmax);
      const bool need = (mcand - m_run) * c2 > kRescaleLog2;
      if (__ballot(need)) {
        const float alpha = need ? exp2f((m_run - mcand) * c2) : 1.0f;
        if (need) m_run = mcand;
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md] *= alpha;
      }
      const float moff = (m_run == kNegInf) ? 0.f : m_run * c2;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = exp2f(__builtin_fmaf(s[i], c2, -moff));
        l_run += s[i];
      }
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          o[md] = mfma32_f32(vt[(8 * (i >> 2) + 4 * h + (i & 3)) * LD + 32 * md + ql], s[i], o[md]);
    }
    __syncthreads();
  }

  const float l_tot = l_run + wave_xor32(l_run);
  if (qi < a.N) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float* O = reinterpret_cast<float*>(a.o) + hoff + (size_t)qi * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = o[md][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(O + 32 * md + 8 * g + 4 * h) = ov;
      }
    if (h == 0) a.lse[(size_t)bh * a.N + qi] = l_tot > 0.f ? m_run * a.sc_abs + logf(l_tot) : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, fa_dtype dt, int d, hipStream_t stream, const KernelTimer& tm) {
  const dim3 grid((unsigned)(a.ntq * a.B * a.H)), block(kThreads);
  if (tm.start) (void)hipEventRecord(tm.start, stream);
  if (dt == FA_BF16) {
    if (d == 64) hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block, 0, stream, a);
  } else {
    if (d == 64) hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (tm.stop) (void)hipEventRecord(tm.stop, stream);
  return e;
}

}  // namespace fa
