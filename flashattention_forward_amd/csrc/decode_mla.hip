// Paged MLA decode for gfx950 over the shared pool [P, page, 576]: the 576-column
// row of a token is its key ([ckv | kpe]) and its first 512 columns its value.
//
// "perf: FlashAttention-3 style MLA PageAttention" (FlashInfer, change list
// items 4 and 5) notes that MLA has one KV stream instead of two, so a single
// load must serve both products and the pipeline needs more, smaller stages to
// keep the next tile's copy in flight while the current one is computed; its
// "Results" section measures batch x seq_len x 64 heads at page_size = 1, where
// every token row is a separate gather. The same ideas, built for CDNA4:
//
//  * a workgroup (4 waves, 16 query heads each, one wave per SIMD) handles one
//    sequence, 64 heads and one key split, so each 1152-byte row leaves HBM
//    once and is read from LDS by both products;
//  * rows are gathered through the page table into registers, two tiles of
//    32 tokens ahead: every lane holds 9 x 16 bytes of each tile in flight,
//    72 KB per CU. (Direct global-to-LDS copies keep far fewer bytes in
//    flight per CU on this hardware and cap a random row gather at about half
//    the HBM rate; plain vector loads do not.) When a tile's turn comes, its
//    lanes write it into a 2-stage LDS ring; one barrier per tile publishes
//    it and retires the stage two tiles back. The page table is resolved once
//    per split into LDS, so no global load in the loop depends on another;
//  * a tile is stored in 8 x 8 blocks of 16-byte chunks (blk_slot): wave w
//    holds token rows 8w .. 8w + 7 and each store moves 8 rows x 128 bytes;
//    the key reads (16 rows of 4 chunks, tokens in the order below) and the
//    transposed value reads (ds_read_b64_tr_b16) are free of bank conflicts;
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32, the LDS reads
//    issued several MFMAs ahead of their use; the running max moves only when
//    it grows by more than 2^8, so the 128 O accumulators per lane are rarely
//    rescaled; row reductions use lane swaps (no LDS);
//  * tokens past the split's end are masked and rows without a valid token
//    (or with a page id out of range) are zeroed in registers before they
//    reach LDS (a NaN in an unused pool slot never reaches the output).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int MLA_DQ = 576;
constexpr int MLA_DV = 512;
constexpr int MLA_ROWB = MLA_DQ * 2;            // 1152 bytes per row
constexpr int MLA_NCH = MLA_DQ / 8;             // 72 chunks of 16 bytes
constexpr int MLA_NST = 2;                      // LDS ring stages
constexpr int MLA_INFL = 2;                     // tiles in flight in registers
constexpr int MLA_STAGE = DEC_TILE * MLA_ROWB;  // 36864 bytes
constexpr int MLA_CPL = DEC_TILE * MLA_NCH / 256;  // 9 chunks per lane and tile
constexpr int MLA_QW = (MLA_DQ / 32) * 1024;   // one wave's query fragments in LDS

// LDS byte offset of chunk c of tile row r: block (r >> 3, c >> 3) of 9 per row band.
__device__ __forceinline__ int mla_slot(int c, int r) {
  return 16 * (64 * (9 * (r >> 3) + (c >> 3)) + blk_slot(r, c));
}

template <typename TI, int PS>
__global__ __launch_bounds__(256, 1) void decode_mla_kernel(DecodeMlaParams p) {
  using T = in_traits<TI>;
  __shared__ __attribute__((aligned(16))) char smem[MLA_NST * MLA_STAGE];
  __shared__ __attribute__((aligned(16))) char qsm[4 * MLA_QW];
  __shared__ int rowid[MLA_MAX_CHUNK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, gq = lane >> 4;

  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int S = p.n_splits;
  const int split = blk % S;
  blk /= S;
  const int hb = blk % p.n_hblk;
  const int b = blk / p.n_hblk;
  const int head = hb * MLA_HEADS_PER_WG + 16 * w + c16;
  const bool hvalid = head < p.Hq;

  const int seq_len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int t0 = split * p.chunk;
  const int n_tok = max(min(p.chunk, seq_len - t0), 0);
  const int n_tiles = (n_tok + DEC_TILE - 1) / DEC_TILE;

  // Resolve the split's page table into pool row ids (-1: page id out of
  // range); all of a thread's page-table loads are issued before any is used.
  {
    const int32_t* ptab = p.page_table + (int64_t)b * p.max_pages;
    constexpr int PER = MLA_MAX_CHUNK / 256;
    int page[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + 256 * k;
      const int key = t0 + i;
      const int pi = PS > 0 ? key / PS : key / p.page_size;
      page[k] = i < n_tok ? ptab[pi] : -1;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + 256 * k;
      if (i < n_tok) {
        const int key = t0 + i;
        const int slot = PS > 0 ? key % PS : key % p.page_size;
        rowid[i] = (unsigned)page[k] < (unsigned)p.num_pages ? page[k] * p.page_size + slot : -1;
      }
    }
  }

  // Query fragments (B operand, 32 dims per MFMA step) live in LDS, each wave's
  // own in lane order (fragment s of lane l at 1024 s + 16 l: conflict-free), so
  // that the registers can hold the tiles in flight.
  char* qw = qsm + MLA_QW * w;
  {
    const char* qrow = (const char*)p.q + ((int64_t)b * p.Hq + (hvalid ? head : 0)) * MLA_ROWB;
    u32x4 qv[MLA_DQ / 32];
#pragma unroll
    for (int s = 0; s < MLA_DQ / 32; ++s)
      qv[s] = hvalid ? ldg16(qrow + (32 * s + 8 * gq) * 2) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < MLA_DQ / 32; ++s)
      *(u32x4*)(qw + 1024 * s + 16 * lane) = p.q_neg ? neg16x8(qv[s]) : qv[s];
  }
  __syncthreads();

  const char* pool = (const char*)p.pool;
  // Lane l of wave w holds chunks 8i + ((l >> 3) ^ (w & 1)) (i < 9) of token row
  // 8w + ((l & 7) ^ 4 * ((l >> 4) & 1)) of every tile: the inverse of blk_slot,
  // so its chunk i goes to byte 1024 (9w + i) + 16 l of the stage.
  const int cp_row = 8 * w + ((lane & 7) ^ (4 * ((lane >> 4) & 1)));
  const int cp_col = 16 * ((lane >> 3) ^ (w & 1));
  const int cp_dst = 1024 * MLA_CPL * w + 16 * lane;
  u32x4 buf[MLA_INFL][MLA_CPL];
  uint32_t badbits = 0;  // bit d: this lane's row of the tile in buf[d] is invalid
  auto load = [&](int t, int d) {
    const int tok = t * DEC_TILE + cp_row;
    const int rid = tok < n_tok ? rowid[tok] : -1;
    badbits = (badbits & ~(1u << d)) | ((rid < 0 ? 1u : 0u) << d);
    const char* src = pool + (int64_t)max(rid, 0) * MLA_ROWB + cp_col;
#pragma unroll
    for (int i = 0; i < MLA_CPL; ++i)
      buf[d][i] = __builtin_nontemporal_load((const u32x4*)(src + 128 * i));
  };
  auto store = [&](int t, int d) {
    char* dst = smem + (t % MLA_NST) * MLA_STAGE + cp_dst;
    const bool bad = (badbits >> d) & 1;
    if (__ballot(bad)) {
#pragma unroll
      for (int i = 0; i < MLA_CPL; ++i)
        *(u32x4*)(dst + 1024 * i) = bad ? u32x4{0, 0, 0, 0} : buf[d][i];
    } else {
#pragma unroll
      for (int i = 0; i < MLA_CPL; ++i) *(u32x4*)(dst + 1024 * i) = buf[d][i];
    }
  };

  f32x4 oacc[MLA_DV / 16];
#pragma unroll
  for (int db = 0; db < MLA_DV / 16; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  // Token order inside a tile. Operand row a (0..15) of score block kb holds
  // token 8 (2 (a >> 3) + kb) + (a & 7): each block takes two row bands of one
  // parity. ds_read_b128 serves the 8-lane groups of a wave in the pairs
  // {0, 3}, {1, 2}, {4, 7}, {5, 6}, and a pair must cover all 64 banks; with
  // this order the two groups of a pair read opposite bank halves. The score
  // S^T[kb][4 gq + i] of a lane is token 16 (gq >> 1) + 8 kb + 4 (gq & 1) + i.
  // Key reads (mla_slot written out): row band 2 (c16 >> 3) + kb, chunk 4s + gq.
  const int kp8 = c16 >> 3;
  const int kswz = 16 * ((c16 & 7) ^ (4 * (gq >> 1)));
  const int koff0 = 18432 * kp8 + 128 * gq + kswz;
  const int koff1 = 18432 * kp8 + 9216 + 128 * (gq ^ 1) + kswz;
  // Transposed value reads, lane j = c16: the PV contraction index 8 gq + k
  // is score row (k >> 2, 4 gq + (k & 3)), so the first read covers tokens
  // 16 (gq >> 1) + 4 (gq & 1) + j / 4 and the second the same + 8, in chunk
  // 2 db + e with e = (j & 3) >> 1, byte 8 (j & 1); the offset alternates with
  // the parity of db.
  const int e = (c16 & 3) >> 1;
  const int tbase = 18432 * (gq >> 1) + 128 * e + 16 * (c16 >> 2) + 8 * (c16 & 1);
  const int toffE = tbase + 64 * (gq & 1), toffO = tbase + 64 * ((gq & 1) ^ 1);
  const int tsecond = 9216 + 128 * (1 - 2 * e);

  constexpr int NQK = 2 * (MLA_DQ / 32), NPV = MLA_DV / 16;
  constexpr int KPD = 6, VPD = 6;  // LDS reads issued this many MFMAs ahead

  // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T. Every wave computes
  // (a wave without valid heads works on zero queries and stores nothing): a
  // branch around the MFMAs would make the compiler shuttle the accumulators
  // between register files. Reads and MFMAs are written out in issue order and
  // fenced so that the order holds.
  auto compute = [&](int t) {
    const char* st = smem + (t % MLA_NST) * MLA_STAGE;
    const int tok0 = t * DEC_TILE;
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
    {
      const char* kp0 = st + koff0;
      const char* kp1 = st + koff1;
      const char* qp = qw + 16 * lane;
      u32x4 kf[NQK], qf[NQK / 2];
      // MFMA i uses key fragment i and query fragment i / 2; read i brings
      // key fragment i and, for even i, query fragment i / 2.
      auto kread = [&](int i) {
        kf[i] = lds16(((i & 1) ? kp1 : kp0) + 512 * (i >> 1));
        if (!(i & 1)) qf[i >> 1] = lds16(qp + 1024 * (i >> 1));
      };
#pragma unroll
      for (int i = 0; i < KPD; ++i) kread(i);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + KPD < NQK) kread(i + KPD);
        sacc[i & 1] = T::mma16(kf[i], qf[i >> 1], sacc[i & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // The first value reads go out before the softmax (they do not depend on it).
    const char* vpE = st + toffE;
    const char* vpO = st + toffO;
    u32x2 va[NPV], vb[NPV];
    auto vread = [&](int db) {
      const char* vp = (db & 1) ? vpO : vpE;
      va[db] = lds_read_tr16(vp + 256 * db);
      vb[db] = lds_read_tr16(vp + 256 * db + tsecond);
    };
#pragma unroll
    for (int i = 0; i < VPD; ++i) vread(i);
    __builtin_amdgcn_sched_barrier(0);
    if (tok0 + DEC_TILE > n_tok) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 16 * (gq >> 1) + 8 * kb + 4 * (gq & 1) + i >= n_tok) sacc[kb][i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mx = max_xor32(max_xor16(mx));
    const bool grow = mx > m_run && (m_run == -INFINITY || (mx - m_run) * sl2 > RESCALE_LOG2);
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * sl2);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < MLA_DV / 16; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float nb = m_run == -INFINITY ? 0.f : -m_run * sl2;
    float pv[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[kb][i] = fast_exp2(fmaf(sacc[kb][i], sl2, nb));
    const u32x4 pb{T::pack2(pv[0][0], pv[0][1]), T::pack2(pv[0][2], pv[0][3]),
                   T::pack2(pv[1][0], pv[1][1]), T::pack2(pv[1][2], pv[1][3])};
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) l_run = T::sum2(pb[q4], l_run);
#pragma unroll
    for (int db = 0; db < NPV; ++db) {
      __builtin_amdgcn_sched_barrier(0);
      if (db + VPD < NPV) vread(db + VPD);
      oacc[db] = T::mma16(u32x4{va[db][0], va[db][1], vb[db][0], vb[db][1]}, pb, oacc[db]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Tile t sits in buf[t % 2]; it is waited for (vmcnt counts the 9 loads of
  // the tile issued after it), stored, its registers reloaded with tile t + 2,
  // published by the barrier and computed. The load schedule is the same on
  // every path, so the compiler's own waits agree with it: loads are always
  // issued (a tile past the split's end reads pool row 0 and is zeroed as
  // invalid) and the loop runs an even number of steps (a padding tile is
  // masked out entirely). The loop is unrolled by two so that every register
  // index is static.
  auto step = [&](int t, int d) {
    wait_vmcnt<MLA_CPL>();
    store(t, d);
    load(t + MLA_INFL, d);
    lds_barrier();
    compute(t);
  };
  load(0, 0);
  load(1, 1);
  for (int t = 0; t < n_tiles; t += MLA_INFL) {
    step(t, 0);
    step(t + 1, 1);
  }
  wait_vmcnt<0>();

  const float l_tot = sum_xor32(sum_xor16(l_run));
  if (!hvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : -INFINITY;
  const int64_t row = (int64_t)b * p.Hq + head;
  if (S == 1) {
    char* orow = (char*)p.o + row * MLA_DV * 2;
#pragma unroll
    for (int db = 0; db < MLA_DV / 16; ++db) {
      const u32x2 v{T::pack2(oacc[db][0] * inv, oacc[db][1] * inv),
                    T::pack2(oacc[db][2] * inv, oacc[db][3] * inv)};
      *(u32x2*)(orow + (16 * db + 4 * gq) * 2) = v;
    }
    if (p.lse && gq == 0) p.lse[row] = lse;
  } else {
    const int64_t rows = (int64_t)p.B * p.Hq;
    float* orow = p.part_o + ((int64_t)split * rows + row) * MLA_DV;
#pragma unroll
    for (int db = 0; db < MLA_DV / 16; ++db)
      *(f32x4*)(orow + 16 * db + 4 * gq) = oacc[db] * inv;
    if (gq == 0) p.part_lse[split * rows + row] = lse;
  }
}

template <typename TI>
static hipError_t mla_dispatch(const DecodeMlaParams& p, hipStream_t stream) {
  const int blocks = p.B * p.n_hblk * p.n_splits;
  if (p.page_size == 1)
    hipLaunchKernelGGL((decode_mla_kernel<TI, 1>), dim3(blocks), dim3(256), 0, stream, p);
  else if (p.page_size == 16)
    hipLaunchKernelGGL((decode_mla_kernel<TI, 16>), dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_mla_kernel<TI, 0>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_mla(const DecodeMlaParams& p, InType it, hipStream_t stream) {
  return it == InType::bf16 ? mla_dispatch<bf16_t>(p, stream) : mla_dispatch<f16_t>(p, stream);
}

}  // namespace fa
