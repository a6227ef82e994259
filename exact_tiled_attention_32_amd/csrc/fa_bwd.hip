// Backward kernels: recompute-based gradients of exact attention (gfx950).
//
// The pages give the principle, not the formulas: the backward recomputes the attention
// tile on chip from Q, K and the saved softmax statistics instead of storing P
// (sendsoonai.com "FlashAttention: IO-aware explained", section "Recomputation and IO
// complexity"; cochat.ai audit of "FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness", quoted App. B.2/B.4). The gradients are the chain rule of
// O = softmax(scale Q K^T) V:
//     P = exp(scale S - lse),  dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//     dK = scale dS^T Q,       dQ = scale dS K,     with D_i = sum_j P_ij dP_ij = dO_i . O_i.
// Loop order follows the quoted Theorem 5 proof (App. C): each key/value tile is loaded
// once and its dK, dV accumulate on chip while query tiles stream past; dQ is read and
// written once per key tile, here as fp32 atomic adds into a workspace accumulator.
//
// Three launches on the caller's stream:
//   1. bwd_pre:     D = rowsum(dO o O) in fp32, and dQ_acc = 0
//   2. bwd_main:    one workgroup per (b, h, 128-key tile); 4 waves, 32 keys each
//   3. bwd_dq_out:  dQ = scale * dQ_acc, rounded to bf16
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;  // keys per workgroup (32 per wave)
// Query rows per inner step: 64 at d = 64; 32 at d = 128, where the register-resident K, V,
// dK^T and dV^T already take 192 registers per lane.
template <int D>
constexpr int query_step() { return D == 128 ? 32 : 64; }

// ---------------------------------------------------------------------------------------
// 1. D = rowsum(dO o O), zero the dQ accumulator. Each thread owns 8 columns of one row.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  const size_t rows = (size_t)a.B * a.H * a.N;
  const size_t gid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t row = gid / LPR;
  const int c0 = (int)(gid % LPR) * 8;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 ov = __builtin_bit_cast(bf16x8, gload16(reinterpret_cast<const __bf16*>(a.o) + row * D + c0));
    const bf16x8 dv = __builtin_bit_cast(bf16x8, gload16(reinterpret_cast<const __bf16*>(a.dout) + row * D + c0));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)ov[e] * (float)dv[e];
    f32x4* dst = reinterpret_cast<f32x4*>(a.dq_acc + row * D + c0);
    dst[0] = f32x4{};
    dst[1] = f32x4{};
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && (gid % LPR) == 0) a.dsum[row] = acc;
}

// Key-tile list helper for the block-sparse path: query tiles [i0, ntq) whose mask block
// in column `cb` is nonzero.
__device__ int build_qtile_list(uint16_t* list, int* wcount, const uint8_t* mask, int cb, int nb,
                                int mb, int i0, int ntq, int bq) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  int count = 0;
  for (int base = i0; base < ntq; base += kThreads) {
    const int i = base + tid;
    const bool keep = i < ntq && mask[(size_t)((i * bq) / mb) * nb + cb] != 0;
    const uint64_t bal = __ballot(keep);
    const int pre = __popcll(bal & ((1ull << l) - 1ull));
    if (l == 0) wcount[w] = __popcll(bal);
    __syncthreads();
    int off = count;
    for (int k = 0; k < w; ++k) off += wcount[k];
    if (keep) list[off + pre] = (uint16_t)i;
    count += wcount[0] + wcount[1] + wcount[2] + wcount[3];
    __syncthreads();
  }
  return count;
}

// ---------------------------------------------------------------------------------------
// 2. Main kernel. Orientation (v_mfma_f32_32x32x16_bf16):
//   S, dP   = Q K^T, dO V^T   (M = queries, N = the wave's 32 keys): K, V rows are
//             register-resident B operands; Q, dO rows are 16-byte LDS reads.
//   dV^T   += dO^T P          (M = d, N = keys): dO^T from transpose reads, P straight
//   dK^T   += Q^T dS           from the accumulator (same layout trick as the forward).
//   dQ     += dS K            (M = queries, N = d, K = the 128 keys of the workgroup):
//             dS goes through LDS as dS^T [key][query]; both operands are transpose
//             reads; the result is added to the fp32 workspace with global atomics.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdArgs a) {
  constexpr int BQ = query_step<D>();
  constexpr int QB = BQ / 32;          // 32-query blocks per step
  constexpr int KS = D / 16;           // k-steps over d
  constexpr int MD = D / 32;           // 32-row blocks of dK^T / dV^T
  constexpr int QT = BQ * D * 2;       // bytes of a Q or dO tile
  constexpr int KT = kBK * D * 2;      // bytes of the K tile
  constexpr int ST = kBK * BQ * 2;     // bytes of the dS^T tile
  constexpr int QCH = BQ * (D / 8) / kThreads;   // 16-byte chunks per thread per Q/dO tile
  constexpr int KCH = kBK * (D / 8) / kThreads;  // 16-byte chunks per thread for K
  // dQ[BQ][D] = dS K has QB * MD = 4 blocks of 32 x 32: one per wave.
  static_assert(QB * MD == 4, "one dQ block per wave");
  __shared__ __attribute__((aligned(16))) char smem[KT + 4 * QT + ST];
  __shared__ __attribute__((aligned(16))) float stats[2][2][BQ];  // [buf][lse2 | D][row]
  __shared__ uint16_t qlist[kMaxTileList];
  __shared__ int wcount[4];

  FA_LDS char* const kt = (FA_LDS char*)smem;
  FA_LDS char* const qbuf = kt + KT;      // [buf][Q | dO]
  FA_LDS char* const st = qbuf + 4 * QT;  // dS^T [128 keys][BQ queries]

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int jt = blockIdx.x / BH;       // key tile; small j (most causal work) first
  const int b = bh / a.H;
  const int k0 = jt * kBK;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, kl = l & 31;
  const int key = k0 + 32 * w + kl;     // the key this lane's accumulator columns refer to
  const size_t hoff = (size_t)bh * a.N * D;
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q) + hoff;
  const __bf16* __restrict__ K = reinterpret_cast<const __bf16*>(a.k) + hoff;
  const __bf16* __restrict__ V = reinterpret_cast<const __bf16*>(a.v) + hoff;
  const __bf16* __restrict__ dO = reinterpret_cast<const __bf16*>(a.dout) + hoff;
  const float* __restrict__ lse = a.lse + (size_t)bh * a.N;
  const float* __restrict__ dsum = a.dsum + (size_t)bh * a.N;
  float* __restrict__ dqa = a.dq_acc + hoff;

  int kv_end = a.N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), a.N);
  const int ntq = (a.N + BQ - 1) / BQ;
  const int i0 = a.causal ? k0 / BQ : 0;
  int nq = k0 < kv_end ? ntq - i0 : 0;  // key tile entirely padded: no work, zero dK/dV
  if (a.mask && nq > 0) nq = build_qtile_list(qlist, wcount, a.mask, k0 / a.mb, a.nb, a.mb, i0, ntq, BQ);

  // Register-resident K and V rows: B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kf[KS], vf[KS];
  {
    const size_t row = (size_t)min(key, a.N - 1) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, gload16(K + row + 16 * ks));
      vf[ks] = __builtin_bit_cast(bf16x8, gload16(V + row + 16 * ks));
      if (key >= a.N) {
        kf[ks] = bf16x8{};
        vf[ks] = bf16x8{};
      }
    }
  }
  // K tile through LDS once, to give each wave the B operand of its dQ block:
  // K[128 keys][32 md_q + l % 32] in the accumulator row order (8 k-steps of 16 keys).
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const int id = tid + kThreads * c;
    const int row = id / (D / 8), col = (id % (D / 8)) * 8;
    const int kk = k0 + row;
    lds_store16(kt + tile_off<D>(row, col), kk < a.N ? gload16(K + (size_t)kk * D + col) : u32x4{});
  }
  const int md_q = w % MD;   // the wave's dQ block: d-block md_q of query block qb_q
  const int qb_q = w / MD;
  __syncthreads();
  bf16x8 kq[kBK / 16];
  {
    int lo, hi;
    tr8_offsets<D>(32 * md_q, lo, hi);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) kq[kk] = lds_tr8(kt + lo + kk * 16 * 2 * D, kt + hi + kk * 16 * 2 * D);
  }

  // Per-lane LDS byte offsets, fixed for the whole kernel.
  int row_off[KS];          // Q / dO row operand: row kl, columns 16 ks + 8h (+32 qb2 rows)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) row_off[ks] = tile_off<D>(kl, 16 * ks + 8 * h);
  int tr_lo[MD], tr_hi[MD];  // Q^T / dO^T transpose reads for d-block md (+16 s4 rows)
#pragma unroll
  for (int md = 0; md < MD; ++md) tr8_offsets<D>(32 * md, tr_lo[md], tr_hi[md]);
  int ds_lo, ds_hi;          // dS^T transpose reads for the wave's dQ query block (+16 kk rows)
  tr8_offsets<BQ>(32 * qb_q, ds_lo, ds_hi);
  // Q / dO tile staging: thread chunk c covers row tid / (D/8) + c * QROWS, column
  // (tid % (D/8)) * 8; QROWS is a multiple of 16, so one swizzled offset serves every chunk.
  const int q_row0 = tid / (D / 8), q_col0 = (tid % (D / 8)) * 8;
  const int qs_off0 = tile_off<D>(q_row0, q_col0);
  constexpr int QROWS = kThreads * 8 / D;
  static_assert(QROWS % 16 == 0, "row step must keep the swizzle");

  f32x16 dkt[MD], dvt[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    dkt[md] = f32x16{};
    dvt[md] = f32x16{};
  }

  // Branch-free load pipeline (see the forward kernel): rows past N read row N-1 and are
  // zeroed when stored; the last step prefetches a valid tile it does not use.
  u32x4 qr[QCH], dr[QCH];
  bool qvalid[QCH];
  float sr = 0.f;
  bool svalid = false;
  auto gload_q = [&](int it) {
    const int q0 = it * BQ;
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      const int qq = q0 + q_row0 + c * QROWS;
      qvalid[c] = qq < a.N;
      const size_t row = (size_t)min(qq, a.N - 1) * D + q_col0;
      qr[c] = gload16(Q + row);
      dr[c] = gload16(dO + row);
    }
    // threads [0, BQ) stage lse (exp2 domain), threads [BQ, 2 BQ) stage D
    const int qq = q0 + (tid & (BQ - 1));
    svalid = qq < a.N;
    const float* src = tid < BQ ? lse : dsum;
    sr = src[min(qq, a.N - 1)];
  };
  auto lds_store_q = [&](int buf) {
    FA_LDS char* qb = qbuf + buf * 2 * QT;
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      lds_store16(qb + qs_off0 + c * QROWS * 2 * D, qvalid[c] ? qr[c] : u32x4{});
      lds_store16(qb + QT + qs_off0 + c * QROWS * 2 * D, qvalid[c] ? dr[c] : u32x4{});
    }
    if (tid < 2 * BQ) {
      float v;
      if (tid < BQ) {
        // an empty row (lse = -inf) and a row past N map to +inf so that P = 0 there
        v = (!svalid || sr == kNegInf) ? __builtin_inff() : sr * kLog2e;
      } else {
        v = svalid ? sr : 0.f;
      }
      stats[buf][tid / BQ][tid & (BQ - 1)] = v;
    }
  };
  // Query tiles are visited last-first: the workgroups of one head that run together
  // then update the same dQ tile at about the same time, so it stays in L2.
  auto tile_at = [&](int t) { return a.mask ? (int)qlist[nq - 1 - t] : i0 + nq - 1 - t; };

  gload_q(nq > 0 ? tile_at(0) : 0);
  lds_store_q(0);
  __syncthreads();

  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    const int it = tile_at(t);
    const int q0 = it * BQ;
    gload_q(tile_at(min(t + 1, nq - 1)));
    const FA_LDS char* qb = qbuf + BUF * 2 * QT;
    const FA_LDS char* db = qb + QT;

    // S = Q K^T and dP = dO V^T for the wave's 32 keys, QB 32-query blocks.
    f32x16 s[QB], dp[QB];
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) {
      s[qb2] = f32x16{};
      dp[qb2] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s[qb2] = mfma32(lds_ld8(qb + row_off[ks] + qb2 * 32 * 2 * D), kf[ks], s[qb2]);
        dp[qb2] = mfma32(lds_ld8(db + row_off[ks] + qb2 * 32 * 2 * D), vf[ks], dp[qb2]);
      }
    }
    // P = exp2(S * scale * log2e - lse * log2e); masked pairs -> 0; dS = P (dP - D).
    const bool edge = (k0 + 32 * w + 31 >= kv_end) || (a.causal && k0 + 32 * w + 31 > q0);
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr0 = 32 * qb2 + 8 * g + 4 * h;
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&stats[BUF][0][qr0]);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(&stats[BUF][1][qr0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          float p = fast_exp2(__builtin_fmaf(s[qb2][i], a.c2s, -l2[e]));
          if (edge && (key >= kv_end || (a.causal && key > q0 + qr0 + e))) p = 0.f;
          s[qb2][i] = p;
          dp[qb2][i] = p * (dp[qb2][i] - dd[e]);
        }
      }
    // dV^T += dO^T P, dK^T += Q^T dS (16 queries per k-step).
#pragma unroll
    for (int s4 = 0; s4 < BQ / 16; ++s4) {
      const bf16x8 pb = pack8(s[s4 >> 1], 8 * (s4 & 1));
      const bf16x8 sb = pack8(dp[s4 >> 1], 8 * (s4 & 1));
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int ro = s4 * 16 * 2 * D;
        dvt[md] = mfma32(lds_tr8(db + tr_lo[md] + ro, db + tr_hi[md] + ro), pb, dvt[md]);
        dkt[md] = mfma32(lds_tr8(qb + tr_lo[md] + ro, qb + tr_hi[md] + ro), sb, dkt[md]);
      }
    }
    // dS^T -> LDS: lane writes 4 consecutive queries of its key per (block, group).
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)dp[qb2][4 * g + e];
        *reinterpret_cast<FA_LDS bf16x4*>(st + tile_off<BQ>(32 * w + kl, 32 * qb2 + 8 * g + 4 * h)) = v4;
      }
    __syncthreads();
    // dQ[q0 .. q0 + BQ)[:] += dS K over the 128 keys: this wave's 32 x 32 block.
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk)
      acc = mfma32(lds_tr8(st + ds_lo + kk * 16 * 2 * BQ, st + ds_hi + kk * 16 * 2 * BQ), kq[kk], acc);
    // Stage the next query tile before issuing the atomics: waiting for its loads then
    // does not also wait for this step's atomics (the memory counter is in-order).
    lds_store_q(BUF ^ 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qq = q0 + 32 * qb_q + 8 * (i >> 2) + 4 * h + (i & 3);
      if (qq < a.N) unsafeAtomicAdd(dqa + (size_t)qq * D + 32 * md_q + kl, acc[i]);
    }
    __syncthreads();
  };
  for (int t = 0; t < nq; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < nq) step(std::integral_constant<int, 1>{}, t + 1);
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane writes 4 consecutive columns of its key.
  if (key < a.N) {
    __bf16* dK = reinterpret_cast<__bf16*>(a.dk) + hoff + (size_t)key * D;
    __bf16* dV = reinterpret_cast<__bf16*>(a.dv) + hoff + (size_t)key * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 kv4, vv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv4[e] = (__bf16)(dkt[md][4 * g + e] * a.scale);
          vv4[e] = (__bf16)dvt[md][4 * g + e];
        }
        *reinterpret_cast<bf16x4*>(dK + 32 * md + 8 * g + 4 * h) = kv4;
        *reinterpret_cast<bf16x4*>(dV + 32 * md + 8 * g + 4 * h) = vv4;
      }
  }
}

// ---------------------------------------------------------------------------------------
// 3. dQ = scale * dQ_acc -> bf16 (8 elements per thread).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void bwd_dq_out_kernel(BwdArgs a, size_t n8) {
  const size_t gid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= n8) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.dq_acc) + 2 * gid;
  const f32x4 x0 = src[0], x1 = src[1];
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)(x0[e] * a.scale);
    r[4 + e] = (__bf16)(x1[e] * a.scale);
  }
  reinterpret_cast<bf16x8*>(a.dq)[gid] = r;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t stream, const KernelTimer& tm) {
  const size_t rows = (size_t)a.B * a.H * a.N;
  const size_t pre_threads = rows * (size_t)(d / 8);
  const dim3 block(kThreads);
  const dim3 gpre((unsigned)((pre_threads + kThreads - 1) / kThreads));
  const dim3 gmain((unsigned)(((a.N + kBK - 1) / kBK) * a.B * a.H));
  const size_t n8 = rows * (size_t)d / 8;
  const dim3 gout((unsigned)((n8 + kThreads - 1) / kThreads));
  if (d == 64) hipLaunchKernelGGL(bwd_pre_kernel<64>, gpre, block, 0, stream, a);
  else hipLaunchKernelGGL(bwd_pre_kernel<128>, gpre, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tm.start) (void)hipEventRecord(tm.start, stream);
  if (d == 64) hipLaunchKernelGGL(bwd_main_kernel<64>, gmain, block, 0, stream, a);
  else hipLaunchKernelGGL(bwd_main_kernel<128>, gmain, block, 0, stream, a);
  e = hipGetLastError();
  if (tm.stop) (void)hipEventRecord(tm.stop, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_out_kernel, gout, block, 0, stream, a, n8);
  return hipGetLastError();
}

}  // namespace fa
