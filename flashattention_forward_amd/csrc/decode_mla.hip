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
//  * a workgroup (8 waves, two per SIMD) handles one sequence, NH = 64 or 32
//    query heads and one key split; each 1152-byte row is read from HBM once
//    per workgroup and from LDS by both products. Waves come in pairs over one
//    group of 16 heads: each computes the partial scores over half of the 576
//    dims, the pair adds its partials through LDS (so both hold the same
//    scores, max and sum) and each accumulates half of the 512 output columns.
//    No MFMA is repeated and a wave holds only half of the query fragments and
//    of the O accumulators. With 64 heads the 4 pairs share every 32-token
//    tile; with 32 heads a step covers 64 tokens, the 2 pairs of waves 0-3 take
//    its first tile and those of waves 4-7 the second, and the two halves'
//    states are merged at the end. The 32-head form lets two workgroups share
//    a sequence's 64 heads without splitting its keys: they run side by side
//    on one XCD, so the second read of each row is served by L2, and no
//    partial results or combine pass are needed;
//  * rows are gathered through the page table into registers a step or two
//    ahead (72-80 KB in flight per CU). (Direct global-to-LDS copies keep far
//    fewer bytes in flight per CU on this hardware and cap a random row gather
//    at about half the HBM rate; plain vector loads do not.) When a step's turn
//    comes its lanes write it into a 2-stage LDS ring; one barrier publishes it
//    and retires the stage two steps back. Every lane loads the page-table
//    entry of its own row two steps ahead of its use, so no global load waits
//    on another inside the loop;
//  * a tile is stored in 8 x 8 blocks of 16-byte chunks (blk_slot), each
//    store moving 8 rows x 128 bytes; the key reads (16 rows of 4 chunks,
//    tokens in the order below) and the transposed value reads
//    (ds_read_b64_tr_b16) are free of bank conflicts;
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32, the LDS reads
//    issued several MFMAs ahead of their use; the running max moves only when
//    it grows by more than 2^8, so the 64 O accumulators per lane are rarely
//    rescaled; row reductions use lane swaps (no LDS);
//  * several new tokens per sequence (Sq > 1) share the workgroup's rows with
//    the heads: row r is new token r % Sq of head r / Sq, so the tokens of a
//    head sit side by side and every row of the workgroup uses each loaded
//    K/V row; token i sees the cached tokens up to position seq_len - Sq + i;
//  * tokens past the split's end are masked and rows without a valid token
//    (or with a page id out of range) are zeroed in registers before they
//    reach LDS (a NaN in an unused pool slot never reaches the output).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int MLA_DQ = 576;
constexpr int MLA_DV = 512;
constexpr int MLA_ROWB = MLA_DQ * 2;            // 1152 bytes per row
constexpr int MLA_TILEB = DEC_TILE * MLA_ROWB;  // 36864 bytes per 32-token tile
constexpr int MLA_NST = 2;                      // LDS ring stages
constexpr int MLA_THREADS = 512;                // 8 waves
constexpr int MLA_QS = MLA_DQ / 32 / 2;         // query fragments per wave (half of the dims)
constexpr int MLA_DVW = MLA_DV / 2;             // output columns per wave

template <int NH> struct MlaCfg {
  static constexpr int NHG = NH / 16;            // head groups (wave pairs per tile)
  // With 64 heads a split's row ids are resolved into LDS once (so a split
  // holds at most MLA_MAX_CHUNK tokens); with 32 heads the ring fills the LDS
  // and every lane loads its row's page-table entry two steps ahead instead.
  static constexpr bool ROWID_LDS = NH == 64;
  static constexpr int TPS = 64 / NH;            // tiles per step
  static constexpr int STEP_TOK = DEC_TILE * TPS;
  static constexpr int INFL = NH == 64 ? 2 : 1;  // steps in flight in registers
  // 16-byte chunks per lane and step: with 64 heads the two waves of a row band
  // take blocks 0-4 and 4-8 of its 9 (both write block 4, with the same bytes);
  // with 32 heads wave w stores row band w of the step's 8.
  static constexpr int CPL = NH == 64 ? 5 : 9;
  static constexpr int STAGE = TPS * MLA_TILEB;
};

template <typename TI, int PS, int NH>
__global__ __launch_bounds__(MLA_THREADS, 2) void decode_mla_kernel(DecodeMlaParams p) {
  using T = in_traits<TI>;
  using C = MlaCfg<NH>;
  constexpr int INFL = C::INFL, CPL = C::CPL;
  __shared__ __attribute__((aligned(16))) char smem[MLA_NST * C::STAGE];
  __shared__ __attribute__((aligned(16))) f32x4 xs[8][2][64];  // partial-score exchange
  __shared__ int rowid[C::ROWID_LDS ? MLA_MAX_CHUNK : 1];        // pool row per token, -1: none
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Head group, half (of the dims and of O) and, with 32 heads, tile of the step.
  const int hg = w % C::NHG, kh = (w / C::NHG) & 1, th = NH == 64 ? 0 : w >> 2;
  const int c16 = lane & 15, gq = lane >> 4;

  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int S = p.n_splits;
  const int split = blk % S;
  blk /= S;
  const int hb = blk % p.n_hblk;
  const int b = blk / p.n_hblk;
  const int rig = hb * NH + 16 * hg + c16;  // row: new token rig % Sq, head rig / Sq
  const int qtok = rig % p.Sq;
  const int head = rig / p.Sq;
  const bool hvalid = head < p.Hq;

  const int seq_len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int t0 = split * p.chunk;
  const int n_tok = max(min(p.chunk, seq_len - t0), 0);
  const int n_steps = (n_tok + C::STEP_TOK - 1) / C::STEP_TOK;
  // Last visible token of this row (split-local) and the smallest over the rows.
  const int lim = min(n_tok - 1, seq_len - p.Sq + qtok - t0);
  const int lim_lo = min(n_tok - 1, seq_len - p.Sq - t0);

  // Staging: lane l of wave w holds chunk 8 cb + ((l >> 3) ^ (rb & 1)) of
  // token row 8 rb + ((l & 7) ^ 4 ((l >> 4) & 1)) of a tile (the inverse of
  // blk_slot), for its blocks cb; block cb of row band rb lives at byte
  // 1024 (9 rb + cb) + 16 l of the tile.
  const int rb = w & 3;
  const int tile_row = 8 * rb + ((lane & 7) ^ (4 * ((lane >> 4) & 1)));
  const int cp_tile = NH == 64 ? 0 : w >> 2;  // tile of the step this wave stores
  const int cb0 = NH == 64 ? 4 * (w >> 2) : 0;
  const int cp_row = DEC_TILE * cp_tile + tile_row;  // token within the step
  const int cp_col = 16 * ((lane >> 3) ^ (rb & 1)) + 128 * cb0;
  const int cp_dst = MLA_TILEB * cp_tile + 1024 * (9 * rb + cb0) + 16 * lane;

  const int32_t* ptab = p.page_table + (int64_t)b * p.max_pages;
  // Page-table entries are read at keys clamped to max_seq_len - 1 (always
  // inside the table, whose rows cover max_seq_len tokens), so these loads do
  // not wait for the sequence length; entries past the split's tokens are
  // ignored. The query loads follow them, so three round trips to memory
  // (length, table, queries) overlap.
  const int key_cap = max(p.max_seq_len - 1, 0);
  constexpr int PER = C::ROWID_LDS ? MLA_MAX_CHUNK / MLA_THREADS : 1;
  int page[PER];
  if constexpr (C::ROWID_LDS) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int key = min(t0 + tid + MLA_THREADS * k, key_cap);
      page[k] = ptab[PS > 0 ? key / PS : key / p.page_size];
    }
  }
  // Pool row (ROWID_LDS) or page-table entry of this lane's row in step s (a
  // token past the split's end reads an entry that exists and is ignored).
  auto pt_load = [&](int s) -> int {
    if constexpr (C::ROWID_LDS) return rowid[min(s * C::STEP_TOK + cp_row, max(n_tok - 1, 0))];
    const int key = min(t0 + s * C::STEP_TOK + cp_row, key_cap);
    return ptab[PS > 0 ? key / PS : key / p.page_size];
  };
  int pg[INFL];
  if constexpr (!C::ROWID_LDS) {
#pragma unroll
    for (int d = 0; d < INFL; ++d) pg[d] = pt_load(d);
  }

  // Query fragments (B operand, 32 dims per MFMA step) of this wave's half of
  // the dims: steps 9 kh .. 9 kh + 8. A wave without valid heads uses head 0's
  // (finite) query and stores nothing.
  u32x4 qf[MLA_QS];
  {
    const char* qrow =
        (const char*)p.q + (((int64_t)b * p.Sq + qtok) * p.Hq + (hvalid ? head : 0)) * MLA_ROWB;
#pragma unroll
    for (int i = 0; i < MLA_QS; ++i) qf[i] = ldg16(qrow + (32 * (MLA_QS * kh + i) + 8 * gq) * 2);
  }
  if constexpr (C::ROWID_LDS) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int key = t0 + tid + MLA_THREADS * k;
      const int slot = PS > 0 ? key % PS : key % p.page_size;
      rowid[tid + MLA_THREADS * k] = tid + MLA_THREADS * k < n_tok &&
                                             (unsigned)page[k] < (unsigned)p.num_pages
                                         ? page[k] * p.page_size + slot
                                         : -1;
    }
    __syncthreads();
#pragma unroll
    for (int d = 0; d < INFL; ++d) pg[d] = pt_load(d);
  }

  const char* pool = (const char*)p.pool;
  u32x4 buf[INFL][CPL];
  uint32_t badbits = 0;  // bit d: this lane's row in buf[d] is invalid
  auto load = [&](int s, int d) {  // rows of step s, from pg[d]
    const int tok = s * C::STEP_TOK + cp_row;
    bool ok;
    int64_t rid;
    if constexpr (C::ROWID_LDS) {
      ok = tok < n_tok && pg[d] >= 0;
      rid = max(pg[d], 0);
    } else {
      const int key = t0 + tok;
      const int slot = PS > 0 ? key % PS : key % p.page_size;
      ok = tok < n_tok && (unsigned)pg[d] < (unsigned)p.num_pages;
      rid = ok ? (int64_t)pg[d] * p.page_size + slot : 0;
    }
    badbits = (badbits & ~(1u << d)) | ((ok ? 0u : 1u) << d);
    const char* src = pool + rid * MLA_ROWB + cp_col;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      buf[d][i] = __builtin_nontemporal_load((const u32x4*)(src + 128 * i));
  };
  auto store = [&](int s, int d) {
    char* dst = smem + (s % MLA_NST) * C::STAGE + cp_dst;
    const bool bad = (badbits >> d) & 1;
    if (__ballot(bad)) {
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        *(u32x4*)(dst + 1024 * i) = bad ? u32x4{0, 0, 0, 0} : buf[d][i];
    } else {
#pragma unroll
      for (int i = 0; i < CPL; ++i) *(u32x4*)(dst + 1024 * i) = buf[d][i];
    }
  };

  f32x4 oacc[MLA_DVW / 16];  // columns 256 kh + 16 db + 4 gq + i
#pragma unroll
  for (int db = 0; db < MLA_DVW / 16; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  // Token order inside a tile. Operand row a (0..15) of score block kb holds
  // token 8 (2 (a >> 3) + kb) + (a & 7): each block takes two row bands of one
  // parity. ds_read_b128 serves the 8-lane groups of a wave in the pairs
  // {0, 3}, {1, 2}, {4, 7}, {5, 6}, and a pair must cover all 64 banks; with
  // this order the two groups of a pair read opposite bank halves. The score
  // S^T[kb][4 gq + i] of a lane is token 16 (gq >> 1) + 8 kb + 4 (gq & 1) + i.
  // Key reads: row band 2 (c16 >> 3) + kb, chunk 4s + gq of the tile.
  const int kp8 = c16 >> 3;
  const int kswz = 16 * ((c16 & 7) ^ (4 * (gq >> 1)));
  const int koff0 = 18432 * kp8 + 128 * gq + kswz + 512 * MLA_QS * kh;
  const int koff1 = 18432 * kp8 + 9216 + 128 * (gq ^ 1) + kswz + 512 * MLA_QS * kh;
  // Transposed value reads, lane j = c16: the PV contraction index 8 gq + k
  // is score row (k >> 2, 4 gq + (k & 3)), so the first read covers tokens
  // 16 (gq >> 1) + 4 (gq & 1) + j / 4 and the second the same + 8, in chunk
  // 2 db + e with e = (j & 3) >> 1, byte 8 (j & 1); the offset alternates with
  // the parity of db.
  constexpr int NQK = 2 * MLA_QS, NPV = MLA_DVW / 16;
  const int e = (c16 & 3) >> 1;
  const int tbase = 18432 * (gq >> 1) + 128 * e + 16 * (c16 >> 2) + 8 * (c16 & 1) + 256 * NPV * kh;
  const int toffE = tbase + 64 * (gq & 1), toffO = tbase + 64 * ((gq & 1) ^ 1);
  const int tsecond = 9216 + 128 * (1 - 2 * e);

  constexpr int KPD = 6, VPD = 6;  // LDS reads issued this many MFMAs ahead

  // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T. Every wave computes
  // (a wave without valid heads works on head 0's query and stores nothing): a
  // branch around the MFMAs would make the compiler shuttle the accumulators
  // between register files. Reads and MFMAs are written out in issue order and
  // fenced so that the order holds.
  auto compute = [&](int s) {
    const char* st = smem + (s % MLA_NST) * C::STAGE + MLA_TILEB * th;
    const int tok0 = (s * C::TPS + th) * DEC_TILE;
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
    {
      const char* kp0 = st + koff0;
      const char* kp1 = st + koff1;
      u32x4 kf[NQK];
      // MFMA i uses key fragment i (score block i & 1, step i >> 1 of this half).
      auto kread = [&](int i) { kf[i] = lds16(((i & 1) ? kp1 : kp0) + 512 * (i >> 1)); };
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
    // Add the partner's partial scores (the other half of the dims).
    xs[w][0][lane] = sacc[0];
    xs[w][1][lane] = sacc[1];
    lds_barrier();
    sacc[0] += xs[w ^ C::NHG][0][lane];
    sacc[1] += xs[w ^ C::NHG][1][lane];
    if (p.q_neg) {  // a negative scale: the scores change sign
      sacc[0] = -sacc[0];
      sacc[1] = -sacc[1];
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
    if (tok0 + DEC_TILE - 1 > lim_lo) {  // past the split's end or a row's position
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 16 * (gq >> 1) + 8 * kb + 4 * (gq & 1) + i > lim) sacc[kb][i] = -INFINITY;
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
      for (int db = 0; db < NPV; ++db) oacc[db] *= alpha;
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

  // Step s sits in buf[s % INFL]; it is waited for (vmcnt counts the loads of
  // the INFL - 1 later steps: CPL rows and one page-table entry each), stored,
  // its registers reloaded with step s + INFL (whose page entries arrived with
  // it), the entries of step s + 2 INFL requested, the stage published by the
  // barrier and computed. The load schedule is the same on every path, so the
  // compiler's own waits agree with it: loads are always issued (rows past the
  // split's end read pool row 0 and are zeroed as invalid) and the loop runs a
  // multiple of INFL steps (a padding step is masked out entirely). The loop
  // is unrolled by INFL so that every register index is static.
  if constexpr (!C::ROWID_LDS)
    wait_vmcnt<MLA_QS>();  // page entries of the first steps (the queries may still be in flight)
#pragma unroll
  for (int d = 0; d < INFL; ++d) {
    load(d, d);
    pg[d] = pt_load(d + INFL);
  }
  auto step = [&](int s, int d) {
    wait_vmcnt<(CPL + !C::ROWID_LDS) * (INFL - 1)>();
    store(s, d);
    load(s + INFL, d);
    pg[d] = pt_load(s + 2 * INFL);
    lds_barrier();
    compute(s);
    debug_step_barrier();
  };
  for (int s = 0; s < n_steps; s += INFL) {
#pragma unroll
    for (int d = 0; d < INFL; ++d) step(s + d, d);
  }
  wait_vmcnt<0>();

  float l_tot = sum_xor32(sum_xor16(l_run));
  if (NH == 32) {
    // Merge the state of the step's second tile (waves 4-7) into that of the
    // first (waves 0-3, same heads and columns) through LDS.
    lds_barrier();  // every wave is done with the stages
    char* xb = smem + (w & 3) * (16 * 1024 + 512);
    if (th == 1) {
#pragma unroll
      for (int db = 0; db < NPV; ++db) *(f32x4*)(xb + 1024 * db + 16 * lane) = oacc[db];
      ((float*)(xb + 16 * 1024))[lane] = m_run;
      ((float*)(xb + 16 * 1024 + 256))[lane] = l_tot;
    }
    lds_barrier();
    if (th == 1) return;
    const float m1 = ((const float*)(xb + 16 * 1024))[lane];
    const float l1 = ((const float*)(xb + 16 * 1024 + 256))[lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m) * sl2);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2((m1 - m) * sl2);
#pragma unroll
    for (int db = 0; db < NPV; ++db)
      oacc[db] = oacc[db] * a0 + *(const f32x4*)(xb + 1024 * db + 16 * lane) * a1;
    l_tot = l_tot * a0 + l1 * a1;
    m_run = m;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : -INFINITY;
  // The output row ([B, Sq, Hq] order), or with several splits this split's
  // partial row (same 16-bit type; the combine weighs the partials by their
  // lse and writes lse as [B, Hq, Sq]). Row rig of the workgroup is new token
  // rig % Sq and head rig / Sq.
  char* obase = (char*)(S == 1 ? p.o : p.part_o) +
                (S == 1 ? 0 : (int64_t)split * p.B * p.Sq * p.Hq * MLA_DV * 2);
  auto out_half = [&](int r) {  // this wave's half of row r's columns
    return obase + ((((int64_t)b * p.Sq + r % p.Sq) * p.Hq + r / p.Sq) * MLA_DV + MLA_DVW * kh) * 2;
  };
  if constexpr (NH == 64) {
    // Through LDS: a lane holds 4 columns of one head per store, so direct
    // stores would touch the wave's 16 rows per instruction. Each wave writes
    // its 16 half rows (512 bytes each; 16-byte chunk q of row j at chunk
    // q ^ j) into its own 8 KB of the idle stages and stores two half rows per
    // instruction.
    lds_barrier();  // every wave is done with the stages
    char* ot = smem + 8192 * w;
#pragma unroll
    for (int db = 0; db < NPV; ++db) {
      const u32x2 v{T::pack2(oacc[db][0] * inv, oacc[db][1] * inv),
                    T::pack2(oacc[db][2] * inv, oacc[db][3] * inv)};
      *(u32x2*)(ot + 512 * c16 + 16 * ((2 * db + (gq >> 1)) ^ c16) + 8 * (gq & 1)) = v;
    }
    wave_lds_sync();
    const int jj = lane >> 5, ch = lane & 31;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 2 * i + jj;
      const u32x4 v = lds16(ot + 512 * j + 16 * (ch ^ j));
      const int r = hb * NH + 16 * hg + j;
      if (r / p.Sq < p.Hq) *(u32x4*)(out_half(r) + 16 * ch) = v;
    }
  } else if (hvalid) {
    char* orow = out_half(rig);
#pragma unroll
    for (int db = 0; db < NPV; ++db) {
      const u32x2 v{T::pack2(oacc[db][0] * inv, oacc[db][1] * inv),
                    T::pack2(oacc[db][2] * inv, oacc[db][3] * inv)};
      *(u32x2*)(orow + (16 * db + 4 * gq) * 2) = v;
    }
  }
  if (hvalid && gq == 0 && kh == 0) {
    const int64_t row = ((int64_t)b * p.Sq + qtok) * p.Hq + head;
    if (S > 1)
      p.part_lse[(int64_t)split * p.B * p.Sq * p.Hq + row] = lse;
    else if (p.lse)
      p.lse[((int64_t)b * p.Hq + head) * p.Sq + qtok] = lse;
  }
}

template <typename TI, int NH>
static hipError_t mla_dispatch_nh(const DecodeMlaParams& p, hipStream_t stream) {
  const int blocks = p.B * p.n_hblk * p.n_splits;
  if (p.page_size == 1)
    hipLaunchKernelGGL((decode_mla_kernel<TI, 1, NH>), dim3(blocks), dim3(MLA_THREADS), 0, stream, p);
  else if (p.page_size == 16)
    hipLaunchKernelGGL((decode_mla_kernel<TI, 16, NH>), dim3(blocks), dim3(MLA_THREADS), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_mla_kernel<TI, 0, NH>), dim3(blocks), dim3(MLA_THREADS), 0, stream, p);
  return hipGetLastError();
}

template <typename TI>
static hipError_t mla_dispatch(const DecodeMlaParams& p, hipStream_t stream) {
  return p.heads_per_wg == 32 ? mla_dispatch_nh<TI, 32>(p, stream) : mla_dispatch_nh<TI, 64>(p, stream);
}

hipError_t launch_decode_mla(const DecodeMlaParams& p, InType it, hipStream_t stream) {
  return it == InType::bf16 ? mla_dispatch<bf16_t>(p, stream) : mla_dispatch<f16_t>(p, stream);
}

}  // namespace fa
