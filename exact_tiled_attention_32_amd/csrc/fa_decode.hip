// Attention of a few queries against a key/value cache, split over the keys (gfx950).
//
// Semantics (aiwiki.page "FlashAttention", section "Software integration and
// limitations", lists inference with cached keys and values among the interfaces): the
// Nq queries of (b, h) are the last Nq positions of a sequence whose first L_b keys and
// values are cached; query i attends key j iff j < L_b and, when causal, j <= L_b - Nq + i.
//
// Decoding reads every cached key and value once and does little arithmetic per byte (it
// is bound by HBM bandwidth), so the work is split over the keys to occupy the whole GPU:
//   1. kvc_split_kernel: each wave owns one "unit", a contiguous range of `chunk` keys of
//      one (b, h), and runs the forward's tiled online softmax over it for all Nq queries
//      (S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, one query per lane,
//      32-key tiles staged by direct buffer -> LDS loads into a ring of LDS stages that
//      belongs to the wave alone, so no workgroup barrier is involved). It writes the
//      unit's partial statistics (m, l) and unnormalised output u = sum_j e^(s_j - m) v_j.
//   2. kvc_merge_kernel: per (b, h, query), combines the units with the online-softmax
//      rule of aiwiki "FlashAttention", section "Tiling and online normalization":
//      m = max_u m_u, l = sum_u e^(m_u - m) l_u, O = sum_u e^(m_u - m) u_u / l, and
//      lse = m + ln l.
#include "fa_device.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {

namespace {

constexpr int kThreads = 256;    // merge kernel
constexpr int kKT = 32;          // keys per tile
constexpr float kRescaleLog2 = 8.0f;
constexpr long long kTargetUnits = 4096;  // key ranges per call, over all (b, h)
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8); the unnamed counters are left free.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xC07F;
// Cache policy of the streaming key/value loads: non-temporal (each byte is read once,
// in whole 16-byte-per-lane rows, so nothing is lost by not keeping it in the caches).
constexpr int kNonTemporal = 2;

// Waves per workgroup (one unit each) and pipeline stages per wave of the key-split
// kernel. A stage holds one K tile and one V tile (2 x 32 x D bf16) in LDS; a wave keeps
// S - 1 tiles in flight while it computes one, so LDS bounds the bytes in flight.
template <int D> struct SplitShape;
template <> struct SplitShape<32> { static constexpr int W = 4, S = 4; };
template <> struct SplitShape<64> { static constexpr int W = 4, S = 4; };
template <> struct SplitShape<128> { static constexpr int W = 3, S = 3; };

// LDS of one pipeline stage of every wave; unused stages shrink to 16 bytes.
template <int D, int STAGE, bool USED = (STAGE < SplitShape<D>::S)>
struct StageLds {
  static constexpr int W = USED ? SplitShape<D>::W : 1;
  static constexpr int BYTES = USED ? 2 * kKT * D * 2 : 16;
};

// DG: head dimension in memory; D: tile width (16 runs on 32-wide tiles, upper half zero).
template <int D, int DG = D>
__global__ __launch_bounds__(SplitShape<D>::W * 64, 1) void kvc_split_kernel(DecArgs a) {
  static_assert(DG == D || (D == 32 && DG == 16), "narrow heads run on 32-wide tiles");
  constexpr int KSG = (DG + 15) / 16;           // k-steps that carry data
  constexpr int W = SplitShape<D>::W;
  constexpr int S = SplitShape<D>::S;
  static_assert(S >= 2 && S <= 4, "pipeline depth");
  constexpr int KS = D / 16;                    // k-steps of the score product
  constexpr int MD = D / 32;                    // 32-row blocks of O^T
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int TILE = kKT * D * 2;             // bytes of a K or V tile
  constexpr int RPB = 1024 / (2 * D);           // tile rows per 1 KB staging block
  constexpr int NB = TILE / 1024;               // staging instructions per tile and tensor
  constexpr int NI = 2 * NB;                    // memory instructions per stage
  // One array per stage, so that the compiler can tell that staging into one stage does
  // not touch the others. Stage layout per wave: [V tile | K tile], both swizzled.
  __shared__ __attribute__((aligned(16))) char st0[StageLds<D, 0>::W][StageLds<D, 0>::BYTES];
  __shared__ __attribute__((aligned(16))) char st1[StageLds<D, 1>::W][StageLds<D, 1>::BYTES];
  __shared__ __attribute__((aligned(16))) char st2[StageLds<D, 2>::W][StageLds<D, 2>::BYTES];
  __shared__ __attribute__((aligned(16))) char st3[StageLds<D, 3>::W][StageLds<D, 3>::BYTES];

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H;
  const int w = wave_id(), l = lane_id(), h = l >> 5, ql = l & 31;
  const int unit = W * (blockIdx.x / BH) + w;
  int L = a.Nk;
  if (a.kv_len) L = min(max(a.kv_len[b], 0), a.Nk);
  const int kb = unit * a.chunk;
  const int ke = min(kb + a.chunk, L);
  const int ntiles = ke > kb ? (ke - kb + kKT - 1) / kKT : 0;

  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q) + (size_t)bh * a.Nq * DG;
  const __bf16* __restrict__ K = reinterpret_cast<const __bf16*>(a.k) + (size_t)bh * a.Nk * DG;
  const __bf16* __restrict__ V = reinterpret_cast<const __bf16*>(a.v) + (size_t)bh * a.Nk * DG;

  // Q fragments (B operand of S^T = K Q^T): lane holds query ql, columns 16 ks + 8 h .. + 7;
  // query rows past Nq are zero (their results are never written). The loads are waited
  // for after the first tiles' loads have been issued.
  u32x4 qraw[KS];
  {
    const __bf16* qrow = Q + (size_t)min(ql, a.Nq - 1) * DG + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks) qraw[ks] = gload16(qrow + 16 * ks);
#pragma unroll
    for (int ks = KSG; ks < KS; ++ks) qraw[ks] = u32x4{};
  }
  bf16x8 qf[KS];

  // LDS operand offsets: K rows (A operand of S^T), V^T transpose reads (A operand of O^T).
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = TILE + tile_off<D>(ql, 16 * ks + 8 * h);
  int v_lo[MD], v_hi[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) tr8_offsets<D>(32 * md, v_lo[md], v_hi[md]);
  // Staging: instruction c writes 1 KB block c (rows c RPB .. + RPB - 1), lane l the 16
  // bytes at 16 l: row c RPB + l / CH, physical chunk l % CH, which holds the logical
  // chunk (l % CH) ^ swz(row).
  int st_off[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int row = c * RPB + l / CH;
    const int chunk = (l % CH) ^ swz<D>(row);
    // a chunk past the head dimension reads zero (offset past any buffer range)
    st_off[c] = 8 * chunk < DG ? (row * DG + chunk * 8) * 2 : (int)0xFFFFFFF0u;
  }
  auto stage = [&](auto si) -> FA_LDS char* {
    if constexpr (decltype(si)::value == 0) return (FA_LDS char*)st0[w];
    else if constexpr (decltype(si)::value == 1) return (FA_LDS char*)st1[w];
    else if constexpr (decltype(si)::value == 2) return (FA_LDS char*)st2[w];
    else return (FA_LDS char*)st3[w];
  };
  // Tile t of the unit into a stage. Rows at or past the unit's end read as zero (buffer
  // range check), so padding never reaches a sum, and a tile wholly past the end makes no
  // memory access at all; it is issued anyway so that every iteration issues the same
  // loads and the waits below stay exact. The wave's LDS reads of the stage (the tile
  // computed last) have returned before new values are written into it.
  auto load = [&](int t, FA_LDS char* dst) {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const int t0 = kb + t * kKT;
    const int rows = __builtin_amdgcn_readfirstlane(t < ntiles ? min(L - t0, kKT) : 0);  // scalar
    const uint32_t bytes = (uint32_t)rows * (uint32_t)(DG * 2);
    const size_t base = t < ntiles ? (size_t)t0 * DG : 0;
    const auto rv = make_rsrc(V + base, bytes);
    const auto rk = make_rsrc(K + base, bytes);
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int voff = st_off[c];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(dst + c * 1024), 16, voff, 0, 0, kNonTemporal);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(dst + TILE + c * 1024), 16, voff, 0, 0,
                                               kNonTemporal);
    }
  };

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;
  const int last = L - a.Nq;  // causal: query i sees keys j <= last + i

  auto tile = [&](const FA_LDS char* vt, int t0) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSG; ++ks) s = mfma32(lds_ld8(vt + k_off[ks]), qf[ks], s);
    // keys past the valid range, or (causal) past a query's position
    if (t0 + kKT > L || (a.causal && t0 + kKT - 1 > last)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t0 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key >= L || (a.causal && key > last + ql)) s[i] = kNegInf;
      }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, other_half(tmax));
    const float mcand = fmaxf(m_run, tmax);
    const bool need = (mcand - m_run) * c2 > kRescaleLog2;
    if (__ballot(need)) {
      const float alpha = need ? fast_exp2((m_run - mcand) * c2) : 1.0f;
      if (need) m_run = mcand;
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < MD; ++md) o[md] *= alpha;
    }
    const float moff = m_run == kNegInf ? 0.f : m_run * c2;
    bf16x8 pb[2];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(__builtin_fmaf(s[i], c2, -moff));
      lsum += p;
      pb[i >> 3][i & 7] = (__bf16)p;
    }
    l_run += lsum;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int md = 0; md < MD; ++md)
        o[md] = mfma32(lds_tr8(vt + v_lo[md] + st * 16 * 2 * D, vt + v_hi[md] + st * 16 * 2 * D), pb[st], o[md]);
  };

  // Ring of S stages: tile t lives in stage t % S; while it is computed, tiles t + 1 ..
  // t + S - 1 are in flight. The loop is unrolled by S so that every stage is a distinct
  // array at every access.
  if (ntiles > 0) {
    load(0, stage(std::integral_constant<int, 0>{}));
    if constexpr (S > 2) load(1, stage(std::integral_constant<int, 1>{}));
    if constexpr (S > 3) load(2, stage(std::integral_constant<int, 2>{}));
    // the Q loads, issued before the tiles', have landed once at most the tiles' remain
    __builtin_amdgcn_s_waitcnt(wait_vmcnt((S - 1) * NI));
    const bool live = ql < a.Nq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, live ? qraw[ks] : u32x4{});
    if (a.qmul != 1.0f) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)qf[ks][e] * a.qmul);
    }
    for (int t = 0; t < ntiles; t += S) {
      auto step = [&](auto j) {
        constexpr int J = decltype(j)::value;
        load(t + J + S - 1, stage(std::integral_constant<int, (J + S - 1) % S>{}));
        __builtin_amdgcn_s_waitcnt(wait_vmcnt((S - 1) * NI));
        if (t + J < ntiles) tile(stage(j), kb + (t + J) * kKT);
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      if constexpr (S > 2) step(std::integral_constant<int, 2>{});
      if constexpr (S > 3) step(std::integral_constant<int, 3>{});
    }
    // the last loads (all past the end) must land before the wave ends
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the unused Q loads
  }

  // Partial results of the unit (an empty unit writes m = -inf, l = 0, u = 0).
  const float l_tot = l_run + other_half(l_run);
  if (ql < a.Nq) {
    const size_t pu = ((size_t)bh * a.units + unit) * a.Nq + ql;
    float* U = a.part_u + pu * DG;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[md][4 * g + e];
        if (32 * md + 8 * g < DG) *reinterpret_cast<f32x4*>(U + 32 * md + 8 * g + 4 * h) = v4;
      }
    if (h == 0) {
      a.part_m[pu] = m_run;
      a.part_l[pu] = l_tot;
    }
  }
}

// One workgroup per (b, h, query). The units are spread over the threads: first the
// maximum of the units' maxima, then groups of D / 4 threads (one 4-column slice each)
// accumulate every G-th unit's weighted output, and the G group sums are added in LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void kvc_merge_kernel(DecArgs a) {
  constexpr int C4 = D / 4;           // threads per output row
  constexpr int G = kThreads / C4;    // unit groups
  __shared__ float wmax[kThreads / 64];
  __shared__ f32x4 gacc[G][C4];
  __shared__ float gl[G];
  const int bh = blockIdx.x / a.Nq, q = blockIdx.x % a.Nq;
  const int tid = threadIdx.x;
  const size_t base = (size_t)bh * a.units * a.Nq + q;  // unit u at base + u Nq
  const int U = a.units;

  float m = kNegInf;
  for (int u = tid; u < U; u += kThreads) m = fmaxf(m, a.part_m[base + (size_t)u * a.Nq]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane_id() == 0) wmax[wave_id()] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

  const int c4 = tid % C4, g = tid / C4;
  f32x4 acc = f32x4{};
  float lsum = 0.f;
  if (m != kNegInf) {
    // an empty unit has m_u = -inf (weight 0), l_u = 0 and u_u = 0
#pragma unroll 4
    for (int u = g; u < U; u += G) {
      const size_t pu = base + (size_t)u * a.Nq;
      const float wgt = fast_exp2((a.part_m[pu] - m) * a.c2);
      lsum += wgt * a.part_l[pu];
      const f32x4 uv = *reinterpret_cast<const f32x4*>(a.part_u + pu * D + 4 * c4);
      acc += wgt * uv;
    }
  }
  gacc[g][c4] = acc;
  if (c4 == 0) gl[g] = lsum;
  __syncthreads();
  if (tid < C4) {
    f32x4 tot = f32x4{};
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      tot += gacc[i][tid];
      lt += gl[i];
    }
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    bf16x4 ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(tot[e] * inv);
    __bf16* O = reinterpret_cast<__bf16*>(a.o) + ((size_t)bh * a.Nq + q) * D + 4 * tid;
    *reinterpret_cast<bf16x4*>(O) = ov;
    if (tid == 0) a.lse[(size_t)bh * a.Nq + q] = lt > 0.f ? m * a.sc_abs + logf(lt) : kNegInf;
  }
}

}  // namespace

void kvcache_split_plan(int B, int H, int Nk, int d, int* chunk, int* units) {
  // about kTargetUnits units in all, each a multiple of the tile; the units of a (b, h)
  // rounded up to whole workgroups
  const int W = kvcache_split_waves(d);
  const long long total = (long long)B * H * Nk;
  long long c = (total + kTargetUnits - 1) / kTargetUnits;
  c = (c + kKT - 1) / kKT * kKT;
  if (c < kKT) c = kKT;
  const long long u = (Nk + c - 1) / c;
  *chunk = (int)c;
  *units = (int)((u + W - 1) / W * W);
}

int kvcache_split_waves(int d) {
  return d <= 32 ? SplitShape<32>::W : d == 64 ? SplitShape<64>::W : SplitShape<128>::W;
}

hipError_t launch_kvcache(const DecArgs& a, int d, hipStream_t stream, KernelTimer& tm) {
  const int W = kvcache_split_waves(d);
  const dim3 gsplit((unsigned)(a.units / W * a.B * a.H)), gmerge((unsigned)(a.B * a.H * a.Nq));
  tm.mark(stream);
  if (d == 16) hipLaunchKernelGGL((kvc_split_kernel<32, 16>), gsplit, dim3(64 * W), 0, stream, a);
  else if (d == 32) hipLaunchKernelGGL(kvc_split_kernel<32>, gsplit, dim3(64 * W), 0, stream, a);
  else if (d == 64) hipLaunchKernelGGL(kvc_split_kernel<64>, gsplit, dim3(64 * W), 0, stream, a);
  else hipLaunchKernelGGL(kvc_split_kernel<128>, gsplit, dim3(64 * W), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tm.mark(stream);
  if (d == 16) hipLaunchKernelGGL(kvc_merge_kernel<16>, gmerge, dim3(kThreads), 0, stream, a);
  else if (d == 32) hipLaunchKernelGGL(kvc_merge_kernel<32>, gmerge, dim3(kThreads), 0, stream, a);
  else if (d == 64) hipLaunchKernelGGL(kvc_merge_kernel<64>, gmerge, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(kvc_merge_kernel<128>, gmerge, dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess) tm.mark(stream);
  return e;
}

}  // namespace fa
