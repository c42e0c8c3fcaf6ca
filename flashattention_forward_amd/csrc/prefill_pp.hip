// Causal / non-causal GQA prefill for gfx950, 8-wave "ping-pong" schedule.
//
// The same tiles, layouts and online softmax as prefill.hip (see there for the
// page references); what differs is how the work of a step is spread over the
// two waves that share a SIMD. With one barrier per step both waves reach their
// copies, waits and softmax at the same moments and the matrix core idles. Here
// the 8 waves form two groups, A (waves 0-3) and B (waves 4-7, one of each per
// SIMD), and every tile is split into two phases:
//   matrix phase M(k): S(k) = K(k) Q^T and O^T += V^T(k-1) P^T(k-1), 32 MFMAs
//                      for head size 128, the LDS reads issued ahead;
//   vector phase V(k): mask, row max, lazy rescale, exp2 / bf16 pack / row sums
//                      of S(k) -> P(k); group B also issues the next copies.
// Group B runs one phase behind group A, and a workgroup barrier separates the
// phases, so while one wave of a SIMD is in a matrix phase the other is in a
// vector phase: the exp-heavy vector work hides under the other wave's MFMAs
// (the FlashAttention-3 overlap that "perf: FlashAttention-3 style MLA
// PageAttention" (FlashInfer, change list item 3) describes, done across two
// waves of one SIMD instead of inside one warpgroup). The wave in its matrix
// phase raises its issue priority.
//
// Phase p = 2k holds A: M(k), B: V(k-1) + copies of K(k+1), V(k); phase
// p = 2k + 1 holds A: V(k), B: M(k) + the wait for those copies. K(j) lives in
// K stage j % 2 and V(j) in V stage j % 2: a stage is refilled in the phase
// after both groups last read it.
//
// Measured on MI355X this schedule matches the single-group interleave of
// prefill.hip (same time on the 512 x 16384 causal microbatch), so it is not
// the default; FA_PREFILL_PINGPONG=1 selects it. S needs one register set (V(k) consumes it before
// M(k+1) overwrites it) and P one (M(k+1) consumes it).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int D> struct PpCfg {
  static constexpr int NCH = D / 8;           // 16-byte chunks per key row
  static constexpr int NCB = NCH / 8;         // 8-chunk blocks per key row
  static constexpr int TILE = PF_BN * D * 2;  // bytes of one K (or V) tile
  static constexpr int NST = 2;               // stages per ring
  static constexpr int LDS = 2 * NST * TILE;  // K ring + V ring
  static constexpr int BM = 256;              // 8 waves x 32 query rows
  static constexpr int BPW = 8 * NCB / 4;     // 1 KB blocks of a tile each group-B wave copies
};

template <int D, typename TI, typename TO, bool CAUSAL>
__global__ __launch_bounds__(512, 2) void prefill_pp_kernel(PrefillParams p) {
  using C = PpCfg<D>;
  using T = in_traits<TI>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wb = w & 3;
  const int c = lane & 31, h = lane >> 5;

  // Logical block: (b, kv head g, query tile, head in group, split), with the
  // blocks that share one K/V head kept on one XCD.
  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int S = p.n_splits;
  const int split = blk % S;
  blk /= S;
  const int G = p.Hq / p.Hkv;
  const int hh = blk % G;
  blk /= G;
  int qt = blk % p.n_qtiles;
  blk /= p.n_qtiles;
  const int g = blk % p.Hkv;
  const int b = blk / p.Hkv;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest rows first
  const int hq = g * G + hh;
  const int off = p.Skv - p.Sq;  // bottom-right alignment
  const int q0 = qt * C::BM;

  int kv_end = p.Skv;
  if (CAUSAL) kv_end = min(kv_end, min(q0 + C::BM, p.Sq) + off);
  const int n_tiles = kv_end > 0 ? (kv_end + PF_BN - 1) / PF_BN : 0;
  const int tps = (n_tiles + S - 1) / S;
  const int t_begin = min(split * tps, n_tiles);
  const int t_end = min(t_begin + tps, n_tiles);
  const int n = t_end - t_begin;

  const int row_bytes = p.Hkv * D * 2;
  const char* kbase = (const char*)p.k + ((int64_t)b * p.Skv * p.Hkv + g) * D * 2;
  const char* vbase = (const char*)p.v + ((int64_t)b * p.Skv * p.Hkv + g) * D * 2;

  // This lane's query row and its Q fragment (B operand, 16 dims per MFMA step).
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + c;
  const bool q_ok = qi < p.Sq;
  u32x4 qf[D / 16];
  {
    const char* qrow = (const char*)p.q + (((int64_t)b * p.Sq + qi) * p.Hq + hq) * D * 2;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 v = q_ok ? ldg16(qrow + (16 * s + 8 * h) * 2) : u32x4{0, 0, 0, 0};
      qf[s] = p.q_neg ? neg16x8(v) : v;
    }
  }

  // Copies (group B only): global_load_lds into the stage, 8 key rows x 128
  // contiguous bytes per instruction. Wave wb of group B copies blocks
  // n = BPW wb + i of a tile (row block RB = n / NCB, chunk block CB = n % NCB):
  // lane l takes chunk 8 CB + ((l >> 3) ^ (RB & 1)) of key row
  // 8 RB + ((l & 7) ^ 4 * ((l >> 4) & 1)) (the inverse of blk_slot). Keys past
  // the end are clamped to the last key (their scores are masked).
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const int dma_rho = (lane & 7) ^ (4 * ((lane >> 4) & 1));
  uint32_t voff[C::BPW];
  int vrow[C::BPW];
#pragma unroll
  for (int i = 0; i < C::BPW; ++i) {
    const int nb = C::BPW * wb + i, RB = nb / C::NCB, cb = nb % C::NCB, rb_odd = RB & 1;
    vrow[i] = 8 * RB + dma_rho;
    voff[i] = (uint32_t)(vrow[i] * row_bytes + (8 * cb + ((lane >> 3) ^ rb_odd)) * 16);
  }
  auto issue = [&](const char* base, uint32_t st, int t) {
    const int k0 = t * PF_BN;
    const char* src = base + (int64_t)k0 * row_bytes;
    const uint32_t dst = st + C::BPW * wb * 1024;
    if (k0 + PF_BN <= p.Skv) {
#pragma unroll
      for (int i = 0; i < C::BPW; ++i) dma16s(src, voff[i], dst + i * 1024);
    } else {
      const int last = p.Skv - 1 - k0;
#pragma unroll
      for (int i = 0; i < C::BPW; ++i) {
        const int over = vrow[i] - last;
        dma16s(src, over > 0 ? voff[i] - (uint32_t)(over * row_bytes) : voff[i], dst + i * 1024);
      }
    }
  };
  auto k_stage = [&](int j) { return (j % C::NST) * C::TILE; };
  auto v_stage = [&](int j) { return (C::NST + (j + C::NST) % C::NST) * C::TILE; };
  auto issue_k = [&](int j) { issue(kbase, smem_lds + k_stage(j), t_begin + j); };
  auto issue_v = [&](int j) { issue(vbase, smem_lds + v_stage(j), t_begin + j); };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  f32x16 sacc[2];
  u32x4 pb[4];
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  // Per-lane LDS offsets (blk_slot written out). K (A operand): row 32 kb + c,
  // chunk 2s + h; the offset alternates with the parity of s.
  const int kbase_off = 1024 * C::NCB * (c >> 3) + 128 * (h ^ ((c >> 3) & 1));
  const int koffE = kbase_off + 16 * (c & 7), koffO = kbase_off + 16 * ((c & 7) ^ 4);
  // V^T (A operand) by transpose reads: lane j = lane & 15 of 16-lane group gb
  // = (lane >> 4) & 1 reads rows 16 jj + 4h + j/4 (read A) and + 8 (read B) of
  // chunk 4 db + 2 gb + e, e = (j & 3) >> 1, byte 8 * (j & 1).
  const int j16 = lane & 15, gb = (lane >> 4) & 1, e = (j16 & 3) >> 1;
  const int voffA = 256 * gb + 128 * e + 64 * (h ^ gb) + 16 * (j16 >> 2) + 8 * (j16 & 1);
  const int voffB = voffA + 1024 * C::NCB + 128 * (1 - 2 * e);

  // Tiles [t_begin, t_mask) are visible to every row of the workgroup and lie
  // inside the keys; the rest (the causal diagonal, the key tail) are masked.
  int t_mask = p.Skv / PF_BN;
  if (CAUSAL)
    t_mask = min(t_mask, q0 + off - (PF_BN - 1) >= 0 ? (q0 + off - (PF_BN - 1)) / PF_BN + 1 : 0);
  const int lim = CAUSAL ? min(p.Skv - 1, qi + off) : p.Skv - 1;

  // Matrix phase: S(k) = K(k) Q^T (QK) and O^T += V^T(k-1) P^T(k-1) (PV), the
  // MFMAs of the two products alternating, each operand read issued a few
  // MFMAs ahead; written out in issue order and fenced.
  constexpr int NQK = D / 8, NPV = D / 8, NDB = D / 32, KPD = 4, VPD = 3;
  auto matrix = [&](auto qk_tag, auto pv_tag, int k) {
    constexpr bool QK = decltype(qk_tag)::value, PV = decltype(pv_tag)::value;
    const char* Ks = smem + k_stage(k);
    const char* Vs = smem + v_stage(k - 1);
    u32x4 kf[NQK];
    u32x2 va[NPV], vb[NPV];
    auto kread = [&](int i) {
      const int s = i >> 1, kb = i & 1;
      kf[i] = lds16(Ks + ((s & 1) ? koffO : koffE) + 256 * s + 4096 * C::NCB * kb);
    };
    auto vread = [&](int i) {
      const int jj = i / NDB, db = i % NDB;
      va[i] = lds_read_tr16(Vs + voffA + 2048 * C::NCB * jj + 512 * db);
      vb[i] = lds_read_tr16(Vs + voffB + 2048 * C::NCB * jj + 512 * db);
    };
    __builtin_amdgcn_s_setprio(1);
    if constexpr (QK) {
#pragma unroll
      for (int i = 0; i < KPD; ++i) kread(i);
    }
    if constexpr (PV) {
#pragma unroll
      for (int i = 0; i < VPD; ++i) vread(i);
    }
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (QK) {
        if (i + KPD < NQK) kread(i + KPD);
        const int s = i >> 1, kb = i & 1;
        sacc[kb] = T::mma32(kf[i], qf[s], s == 0 ? f32x16{} : sacc[kb]);
      }
      if constexpr (PV) {
        if (i + VPD < NPV) vread(i + VPD);
        const int jj = i / NDB, db = i % NDB;
        oacc[db] = T::mma32(u32x4{va[i][0], va[i][1], vb[i][0], vb[i][1]}, pb[jj], oacc[db]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  // Vector phase: S(k) -> P(k). Masked tiles get -inf beyond `lim` first; the
  // running max moves only when it grows by > 2^8. exp2(-inf * sl2 + nb) = 0
  // because sl2 > 0 (a zero scale is passed as the smallest positive one).
  auto vector = [&](int k) {
    const int t = t_begin + k;
    if (t >= t_mask) {
      const int k0 = t * PF_BN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key > lim) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = max_xor32(mx);
    const bool grow = mx > m_run && (m_run == -INFINITY || (mx - m_run) * sl2 > RESCALE_LOG2);
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * sl2);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float nb = m_run == -INFINITY ? 0.f : -m_run * sl2;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int kb = jj >> 1, base = 8 * (jj & 1);
      float pv[8];
#pragma unroll
      for (int ee = 0; ee < 8; ++ee) pv[ee] = fast_exp2(fmaf(sacc[kb][base + ee], sl2, nb));
      pb[jj] = u32x4{T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3]), T::pack2(pv[4], pv[5]),
                     T::pack2(pv[6], pv[7])};
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) l_run = T::sum2(pb[jj][q4], l_run);
    }
  };

  constexpr std::integral_constant<bool, true> kOn{};
  constexpr std::integral_constant<bool, false> kOff{};
  // Each group runs its own loop; both execute the same sequence of
  // workgroup barriers (s_barrier counts waves, not program counters).
  if (n > 0) {
    if (grp == 0) {
      lds_barrier();  // K(0) copied
      matrix(kOn, kOff, 0);
      lds_barrier();
      vector(0);
      lds_barrier();
      for (int k = 1; k < n; ++k) {
        matrix(kOn, kOn, k);
        lds_barrier();
        vector(k);
        lds_barrier();
      }
      matrix(kOff, kOn, n);
      lds_barrier();
    } else {
      issue_k(0);
      wait_vmcnt<0>();
      lds_barrier();
      if (1 < n) issue_k(1);
      issue_v(0);
      lds_barrier();
      matrix(kOn, kOff, 0);
      wait_vmcnt<0>();
      lds_barrier();
      for (int k = 1; k < n; ++k) {
        vector(k - 1);
        if (k + 1 < n) issue_k(k + 1);
        issue_v(k);
        lds_barrier();
        matrix(kOn, kOn, k);
        wait_vmcnt<0>();
        lds_barrier();
      }
      vector(n - 1);
      lds_barrier();
      matrix(kOff, kOn, n);
    }
  }

  // Epilogue: both lane halves hold parts of the row sum.
  const float l_tot = sum_xor32(l_run);
  if (!q_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : -INFINITY;
  // The output row, or with several splits this split's partial row (in the
  // output's type; the combine weighs the partials by their lse).
  const int64_t row = ((int64_t)b * p.Sq + qi) * p.Hq + hq;
  const int64_t prow = S == 1 ? row : (int64_t)split * p.B * p.Sq * p.Hq + row;
  char* orow = (char*)(S == 1 ? p.o : p.part_o) + prow * D * out_size<TO>::bytes;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * db + 8 * i4 + 4 * h;
      store4(TO{}, orow + d * out_size<TO>::bytes, oacc[db][4 * i4] * inv,
             oacc[db][4 * i4 + 1] * inv, oacc[db][4 * i4 + 2] * inv,
             oacc[db][4 * i4 + 3] * inv);
    }
  if (h == 0) {
    if (S == 1) {
      if (p.lse) p.lse[((int64_t)b * p.Hq + hq) * p.Sq + qi] = lse;
    } else {
      p.part_lse[prow] = lse;
    }
  }
}

template <int D, typename TI, typename TO>
static hipError_t launch_pp3(const PrefillParams& p, bool causal, hipStream_t stream) {
  const int n = p.B * p.Hq * p.n_qtiles * p.n_splits;
  if (causal)
    hipLaunchKernelGGL((prefill_pp_kernel<D, TI, TO, true>), dim3(n), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_pp_kernel<D, TI, TO, false>), dim3(n), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <typename TI>
static hipError_t launch_pp2(const PrefillParams& p, OutType ot, bool causal, hipStream_t stream) {
  switch (ot) {
    case OutType::bf16: return launch_pp3<128, TI, out_bf16>(p, causal, stream);
    case OutType::f16: return launch_pp3<128, TI, out_f16>(p, causal, stream);
    default: return launch_pp3<128, TI, out_f32>(p, causal, stream);
  }
}

hipError_t launch_prefill_pp(const PrefillParams& p, InType it, OutType ot, bool causal,
                             hipStream_t stream) {
  return it == InType::bf16 ? launch_pp2<bf16_t>(p, ot, causal, stream)
                            : launch_pp2<f16_t>(p, ot, causal, stream);
}

}  // namespace fa
