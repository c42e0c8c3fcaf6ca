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
//  * a workgroup (4 waves, 16 query heads each) handles one sequence, 64 heads
//    and one key split, so each 1152-byte row leaves HBM once and is read from
//    LDS by both products;
//  * rows are gathered through the page table straight into LDS with
//    global_load_lds_dwordx4 (no VGPR staging) into a 4-stage ring: three tiles
//    of 32 tokens are in flight while one is computed. The page table is
//    resolved once per split into LDS, so no global load in the loop depends on
//    another. Barriers wait on LDS only; each wave waits (vmcnt) for its own
//    copies of the tile it is about to use;
//  * a tile is stored in 8 x 8 blocks of 16-byte chunks (blk_slot): one copy
//    instruction moves 8 token rows x 128 contiguous bytes, wave w copies token
//    rows 8w .. 8w + 7 (each lane the same row in all 9 of its copies), and both
//    the key reads (16 rows of one chunk) and the transposed value reads
//    (ds_read_b64_tr_b16: 8 rows x 2 chunks) touch 64 distinct banks;
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32 as in the other
//    decode kernel; the running max moves only when it grows by more than 2^8,
//    so the 128 O accumulators per lane are rarely rescaled;
//  * tokens past the sequence end are masked and their LDS rows zero-filled (a
//    NaN in an unused pool slot never reaches the output).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int MLA_DQ = 576;
constexpr int MLA_DV = 512;
constexpr int MLA_ROWB = MLA_DQ * 2;               // 1152 bytes per row
constexpr int MLA_NCH = MLA_DQ / 8;                // 72 chunks of 16 bytes
constexpr int MLA_NST = 4;                         // LDS ring stages
constexpr int MLA_STAGE = DEC_TILE * MLA_ROWB;     // 36864 bytes
constexpr int MLA_IPW = DEC_TILE * MLA_NCH / 64 / 4;  // 9 copy instructions per wave and tile

// LDS byte offset of chunk c of tile row r: block (r >> 3, c >> 3) of 9 per row band.
__device__ __forceinline__ int mla_slot(int c, int r) {
  return 16 * (64 * (9 * (r >> 3) + (c >> 3)) + blk_slot(r, c));
}

template <typename TI, int PS>
__global__ __launch_bounds__(256, 1) void decode_mla_kernel(DecodeMlaParams p) {
  using T = in_traits<TI>;
  __shared__ __attribute__((aligned(16))) char smem[MLA_NST * MLA_STAGE];
  __shared__ int rowid[MLA_MAX_CHUNK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

  // Query fragments: B operand, 32 dims per MFMA step.
  u32x4 qf[MLA_DQ / 32];
  {
    const char* qrow = (const char*)p.q + ((int64_t)b * p.Hq + (hvalid ? head : 0)) * MLA_ROWB;
#pragma unroll
    for (int s = 0; s < MLA_DQ / 32; ++s) {
      const u32x4 v = hvalid ? ldg16(qrow + (32 * s + 8 * gq) * 2) : u32x4{0, 0, 0, 0};
      qf[s] = p.q_neg ? neg16x8(v) : v;
    }
  }

  // Resolve the split's page table into pool row ids (-1: page id out of range).
  {
    const int32_t* ptab = p.page_table + (int64_t)b * p.max_pages;
    for (int i = tid; i < n_tok; i += 256) {
      int pi, slot;
      const int key = t0 + i;
      if (PS > 0) {
        pi = key / PS;
        slot = key % PS;
      } else {
        pi = key / p.page_size;
        slot = key - pi * p.page_size;
      }
      const int page = ptab[pi];
      rowid[i] = (unsigned)page < (unsigned)p.num_pages ? page * p.page_size + slot : -1;
    }
  }
  __syncthreads();

  const char* pool = (const char*)p.pool;
  const uint32_t smem_lds = lds_addr(smem);
  // Copy tile t into stage t % MLA_NST. Instruction i of wave w fills block
  // (w, i): lane l copies chunk 8i + ((l >> 3) ^ (w & 1)) of token row
  // 8w + ((l & 7) ^ 4 * ((l >> 4) & 1)) (the inverse of blk_slot). Every wave
  // issues exactly MLA_IPW copies per tile (the vmcnt waits count on it); rows
  // without a valid token read pool row 0 and are zeroed before use.
  const int dma_row = 8 * w + ((lane & 7) ^ (4 * ((lane >> 4) & 1)));
  const int dma_col = 16 * ((lane >> 3) ^ (w & 1));
  auto issue = [&](int t) {
    const uint32_t dst = smem_lds + (t % MLA_NST) * MLA_STAGE + MLA_IPW * w * 1024;
    const int tok = t * DEC_TILE + dma_row;
    int rid = tok < n_tok ? rowid[tok] : -1;
    rid = rid < 0 ? 0 : rid;
    const char* src = pool + (int64_t)rid * MLA_ROWB + dma_col;
#pragma unroll
    for (int i = 0; i < MLA_IPW; ++i) dma16(src + 128 * i, dst + 1024 * i);
  };

  f32x4 oacc[MLA_DV / 16];
#pragma unroll
  for (int db = 0; db < MLA_DV / 16; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  // Key reads: rows 16 * kb + c16 of chunk 4s + gq (mla_slot written out).
  const int kp8 = c16 >> 3;
  const int koff = 9216 * kp8 + 128 * (gq ^ kp8) + 16 * ((c16 & 7) ^ (4 * (gq >> 1)));
  // Transposed value reads, lane j = c16: rows 4gq + j/4 (and +16) of chunk
  // 2db + e with e = (j & 3) >> 1, byte 8 * (j & 1) inside the chunk; the offset
  // alternates with the parity of db.
  const int e = (c16 & 3) >> 1;
  const int tbase = 9216 * (gq >> 1) + 128 * (e ^ ((gq >> 1) & 1)) + 16 * (c16 >> 2) + 8 * (c16 & 1);
  const int toffE = tbase + 64 * (gq & 1), toffO = tbase + 64 * ((gq & 1) ^ 1);

  for (int t = 0; t < min(n_tiles, MLA_NST - 1); ++t) issue(t);

  for (int t = 0; t < n_tiles; ++t) {
    if (t + 2 < n_tiles)
      wait_vmcnt<2 * MLA_IPW>();
    else if (t + 1 < n_tiles)
      wait_vmcnt<MLA_IPW>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    char* st = smem + (t % MLA_NST) * MLA_STAGE;
    const int tok0 = t * DEC_TILE;
    // Rows without a valid token (tail of the split, bad page id) -> zeros.
    {
      const int r = lane & 31;
      const bool bad = tok0 + r >= n_tok || rowid[tok0 + r] < 0;
      const uint64_t badmask = __ballot(bad) & 0xffffffffull;
      if (badmask) {
        for (int i = tid; i < DEC_TILE * MLA_NCH; i += 256) {
          const int rr = i / MLA_NCH, cc = i - rr * MLA_NCH;
          if ((badmask >> rr) & 1) *(u32x4*)(st + mla_slot(cc, rr)) = u32x4{0, 0, 0, 0};
        }
        lds_barrier();
      }
    }
    if (t + MLA_NST - 1 < n_tiles) issue(t + MLA_NST - 1);

    // Every wave computes (a wave without valid heads works on zero queries
    // and stores nothing): a branch around the MFMAs would make the compiler
    // shuttle the accumulators between register files.
    {
      f32x4 sacc[2] = {f32x4{}, f32x4{}};
      const char* kp = st + koff;
#pragma unroll
      for (int s = 0; s < MLA_DQ / 32; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a = lds16(kp + 512 * s + 18432 * kb);
          sacc[kb] = T::mma16(a, qf[s], sacc[kb]);
        }
      }
      if (tok0 + DEC_TILE > n_tok) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tok0 + 16 * kb + 4 * gq + i >= n_tok) sacc[kb][i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                       fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
      mx = fmaxf(mx, xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const bool grow = mx > m_run && (m_run == -INFINITY || (mx - m_run) * sl2 > RESCALE_LOG2);
      if (__ballot(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * sl2);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < MLA_DV / 16; ++db) acc_scale(oacc[db], alpha);
        m_run = m_new;
      }
      const float nb = m_run == -INFINITY ? 0.f : -m_run * sl2;
      float pv[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[kb][i] = fast_exp2(fmaf(sacc[kb][i], sl2, nb));
          l_run += pv[kb][i];
        }
      const u32x4 pb{T::pack2(pv[0][0], pv[0][1]), T::pack2(pv[0][2], pv[0][3]),
                     T::pack2(pv[1][0], pv[1][1]), T::pack2(pv[1][2], pv[1][3])};
      const char* vpE = st + toffE;
      const char* vpO = st + toffO;
#pragma unroll
      for (int db = 0; db < MLA_DV / 16; ++db) {
        const char* vp = (db & 1) ? vpO : vpE;
        const u32x2 r0 = lds_read_tr16(vp + 256 * db);
        const u32x2 r1 = lds_read_tr16(vp + 256 * db + 18432);
        oacc[db] = T::mma16(u32x4{r0[0], r0[1], r1[0], r1[1]}, pb, oacc[db]);
      }
    }
  }

  float l_tot = l_run + xor16(l_run);
  l_tot += xor32(l_tot);
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
