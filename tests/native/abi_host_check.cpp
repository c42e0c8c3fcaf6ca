// Host-only check of the C-ABI front end (csrc/api.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer. Test infrastructure: built with g++ by
// tests/test_host_sanitizers.py together with api.cpp, with no GPU code.
//
// The HIP runtime calls the front end makes and the kernel launchers are
// replaced here by host stubs. A launcher stub checks the parameter block
// against what the kernel assumes (tile counts cover the rows, head packs
// divide the groups, split chunks cover the keys, grids fit) and then writes
// every byte of workspace the kernel would write and the combine would read.
// The workspace is a host allocation of exactly the size the matching
// *_workspace_size query returned, so a plan that needs more than the query
// promised is a heap overflow that ASan reports.
//
// Modes: "sweep" runs every shape / override sweep and prints "checked N
// calls"; "log" makes a few calls (run it with FA_LOG=1 to see the plan lines).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "fa.h"
#include "fa_kernels.h"

namespace {

int g_failures = 0;
long g_calls = 0;
int g_stub_cus = 96;  // what the stubbed device reports

#define CHECK(cond, ...)                                               \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                               \
      std::fprintf(stderr, "\n");                                      \
      if (++g_failures > 20) std::exit(1);                             \
    }                                                                  \
  } while (0)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Counters of what the stubs saw in the current call.
struct Seen {
  int prefill = 0, combine = 0, dsplit = 0, dmla = 0;
  int waves = 0, pack = 0, splits = 0;
};
Seen g_seen;

// Whether the current call's workspace is a real host allocation.
bool g_touch = true;

// Touch [p, p + n) as the kernels would (writes, then reads back).
void touch(void* p, size_t n) {
  if (n == 0 || !g_touch) return;
  std::memset(p, 0x5a, n);
  volatile unsigned char acc = 0;
  const unsigned char* c = (const unsigned char*)p;
  for (size_t i = 0; i < n; i += 4096) acc ^= c[i];
  acc ^= c[n - 1];
  (void)acc;
}

// A device address stand-in: aligned, never dereferenced by the front end.
void* fake(uintptr_t tag) { return reinterpret_cast<void*>(tag << 12); }

void* g_scratch = nullptr;  // host stand-in of the static decode scratch

}  // namespace

// ---------------------------------------------------------------------------
// HIP runtime stubs (the only runtime calls api.cpp makes).
// ---------------------------------------------------------------------------
extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* pi, hipDeviceAttribute_t attr, int deviceId) {
  if (attr != hipDeviceAttributeMultiprocessorCount || deviceId != 0) return hipErrorInvalidValue;
  *pi = g_stub_cus;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
}

// ---------------------------------------------------------------------------
// Launcher stubs.
// ---------------------------------------------------------------------------
namespace fa {

hipError_t launch_prefill(const PrefillParams& p, int D, InType, OutType ot, bool,
                          hipStream_t) {
  g_seen.prefill++;
  g_seen.waves = p.waves;
  g_seen.pack = p.pack;
  g_seen.splits = p.n_splits;
  const int G = p.Hq / p.Hkv;
  CHECK(p.waves == 4 || p.waves == 8, "waves %d", p.waves);
  CHECK(p.waves == 4 || D == 128, "8 waves with D=%d", D);
  CHECK(p.pack >= 1 && p.waves % p.pack == 0 && G % p.pack == 0, "pack %d waves %d G %d",
        p.pack, p.waves, G);
  CHECK(!p.pingpong || p.pack == 1 || p.waves != 8, "ping-pong with a head pack");
  const int rows_per_tile = 32 * p.waves / p.pack;
  CHECK((int64_t)p.n_qtiles * rows_per_tile >= p.Sq, "qtiles %d x %d < Sq %d", p.n_qtiles,
        rows_per_tile, p.Sq);
  CHECK((int64_t)(p.n_qtiles - 1) * rows_per_tile < p.Sq, "idle query tile");
  CHECK(p.n_splits >= 1 && p.n_splits <= 64, "splits %d", p.n_splits);
  CHECK(p.n_splits == 1 || p.n_splits <= cdiv(p.Skv, PF_BN), "more splits than key tiles");
  const int64_t grid = (int64_t)p.B * (p.Hq / p.pack) * p.n_qtiles * p.n_splits;
  CHECK(grid >= 1 && grid <= 0x7fffffff, "grid %lld", (long long)grid);
  CHECK(p.scale >= 0.f && p.scale_log2 > 0.f && std::isfinite(p.scale_log2), "scale");
  if (p.mask) {
    CHECK(p.mask_stride % 8 == 0 && p.mask_stride >= cdiv(p.Skv, 8) * 8, "mask stride");
    CHECK(p.mask_bstride % 8 == 0 && p.mask_bstride >= 0, "mask batch stride");
  }
  if (p.n_splits > 1) {
    const int64_t rows = (int64_t)p.B * p.Sq * p.Hq;
    const size_t ob = ot == OutType::f32 ? 4 : 2;
    CHECK(p.part_o && p.part_lse, "split without partial buffers");
    CHECK(((uintptr_t)p.part_o & 15) == 0 && ((uintptr_t)p.part_lse & 15) == 0,
          "partials not 16-byte aligned");
    CHECK((char*)p.part_lse == (char*)p.part_o + p.n_splits * rows * D * ob,
          "lse partials do not follow the row partials");
    touch(p.part_o, (size_t)p.n_splits * rows * D * ob);
    touch(p.part_lse, (size_t)p.n_splits * rows * sizeof(float));
  }
  return hipSuccess;
}

hipError_t launch_combine(const CombineParams& c, OutType, hipStream_t) {
  g_seen.combine++;
  CHECK(c.n_splits > 1, "combine of %d splits", c.n_splits);
  CHECK(c.rows > 0, "rows");
  CHECK(c.rows % (c.Sq * c.Hq) == 0, "rows %d not a multiple of Sq*Hq", c.rows);
  const size_t pb = c.part16 ? 2 : 4;
  touch(const_cast<void*>(c.part_o), (size_t)c.n_splits * c.rows * c.D * pb);
  touch(const_cast<float*>(c.part_lse), (size_t)c.n_splits * c.rows * sizeof(float));
  return hipSuccess;
}

static void check_split_cover(int chunk, int n_splits, int max_seq_len) {
  CHECK(chunk > 0 && chunk % DEC_TILE == 0, "chunk %d", chunk);
  CHECK((int64_t)chunk * n_splits >= max_seq_len, "splits do not cover the keys");
  CHECK((int64_t)chunk * (n_splits - 1) < std::max(1, max_seq_len), "an empty split");
}

hipError_t launch_decode_split(const DecodeSplitParams& p, InType, hipStream_t) {
  g_seen.dsplit++;
  g_seen.splits = p.n_splits;
  const int G = p.Hq / p.Hkv;
  CHECK((int64_t)p.n_hblk * 16 >= (int64_t)p.Sq * G, "row blocks");
  CHECK((int64_t)(p.n_hblk - 1) * 16 < (int64_t)p.Sq * G, "idle row block");
  CHECK((int64_t)p.n_units == (int64_t)p.B * p.Hkv * p.n_hblk * p.n_splits, "units");
  check_split_cover(p.chunk, p.n_splits, p.max_seq_len);
  if (p.n_splits > 1) {
    const int64_t rows = (int64_t)p.B * p.Sq * p.Hq;
    CHECK((char*)p.part_lse == (char*)p.part_o + p.n_splits * rows * 128 * 2, "lse offset");
    touch(p.part_o, (size_t)p.n_splits * rows * 128 * 2);
    touch(p.part_lse, (size_t)p.n_splits * rows * sizeof(float));
  }
  return hipSuccess;
}

hipError_t launch_decode_mla(const DecodeMlaParams& p, InType, hipStream_t) {
  g_seen.dmla++;
  g_seen.splits = p.n_splits;
  CHECK(p.heads_per_wg == 32 || p.heads_per_wg == 64, "heads %d", p.heads_per_wg);
  CHECK((int64_t)p.n_hblk * p.heads_per_wg >= (int64_t)p.Hq * p.Sq, "head blocks");
  CHECK((int64_t)(p.n_hblk - 1) * p.heads_per_wg < (int64_t)p.Hq * p.Sq, "idle head block");
  CHECK(p.heads_per_wg == 32 || p.chunk <= MLA_MAX_CHUNK, "64-head chunk %d > %d", p.chunk,
        MLA_MAX_CHUNK);
  check_split_cover(p.chunk, p.n_splits, p.max_seq_len);
  CHECK((int64_t)p.B * p.n_hblk * p.n_splits <= 0x7fffffff, "grid");
  if (p.n_splits > 1) {
    const int64_t rows = (int64_t)p.B * p.Sq * p.Hq;
    CHECK((char*)p.part_lse == (char*)p.part_o + p.n_splits * rows * 512 * 2, "lse offset");
    touch(p.part_o, (size_t)p.n_splits * rows * 512 * 2);
    touch(p.part_lse, (size_t)p.n_splits * rows * sizeof(float));
  }
  return hipSuccess;
}

hipError_t device_scratch(void** ptr) {
  if (!g_scratch) g_scratch = std::malloc(NOALLOC_SCRATCH_BYTES);
  *ptr = g_scratch;
  return g_scratch ? hipSuccess : hipErrorOutOfMemory;
}

}  // namespace fa

// ---------------------------------------------------------------------------
// Sweeps.
// ---------------------------------------------------------------------------
namespace {

// Exact-size host workspace (nullptr for 0 bytes), 16-byte aligned by malloc.
struct Buf {
  void* p = nullptr;
  explicit Buf(size_t n) {
    if (n) p = std::malloc(n);
  }
  ~Buf() { std::free(p); }
};

// Larger plans get a stand-in address and the arithmetic checks only.
constexpr size_t kMaxTouch = (size_t)4 << 20;

// Exact-size workspace, or a stand-in address for one above kMaxTouch.
struct Workspace {
  Buf buf;
  void* p;
  explicit Workspace(size_t n) : buf(n <= kMaxTouch ? n : 0), p(n <= kMaxTouch ? buf.p : fake(7)) {
    g_touch = n <= kMaxTouch;
  }
};

void set_env(const char* name, int v) {
  if (v == 0)
    unsetenv(name);
  else
    setenv(name, std::to_string(v).c_str(), 1);
}

void prefill_case(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal, fa_dtype od,
                  bool mask) {
  const size_t ws = fa_prefill_workspace_size(B, Hq, Hkv, Sq, Skv, D, causal, od);
  Workspace w(ws);
  g_seen = Seen{};
  const int64_t ms = cdiv(std::max(Skv, 1), 8) * 8;
  int rc;
  if (mask)
    rc = fa_prefill_mask(fake(1), fake(2), fake(3), fake(4), ms, 0, fake(5), (float*)fake(6), B,
                         Hq, Hkv, Sq, Skv, D, causal, 0.088f, FA_BF16, od, w.p, ws, nullptr);
  else
    rc = fa_prefill_ex(fake(1), fake(2), fake(3), fake(5), (float*)fake(6), B, Hq, Hkv, Sq, Skv,
                       D, causal, 0.088f, FA_BF16, od, w.p, ws, nullptr);
  ++g_calls;
  CHECK(rc == FA_OK, "prefill rc %d B%d Hq%d Hkv%d Sq%d Skv%d D%d", rc, B, Hq, Hkv, Sq, Skv, D);
  if (rc != FA_OK) return;
  CHECK(g_seen.prefill == (Sq > 0), "launches %d", g_seen.prefill);
  CHECK(g_seen.combine == (g_seen.splits > 1 ? 1 : 0), "combine %d splits %d", g_seen.combine,
        g_seen.splits);
  CHECK((ws > 0) == (g_seen.splits > 1) || Sq == 0, "workspace %zu with %d splits", ws,
        g_seen.splits);
  // Without a workspace the same shape never splits.
  g_seen = Seen{};
  rc = fa_prefill_ex(fake(1), fake(2), fake(3), fake(5), nullptr, B, Hq, Hkv, Sq, Skv, D, causal,
                     0.088f, FA_BF16, od, nullptr, 0, nullptr);
  ++g_calls;
  CHECK(rc == FA_OK && g_seen.combine == 0 && (Sq == 0 || g_seen.splits == 1),
        "no-workspace call rc %d splits %d", rc, g_seen.splits);
}

void prefill_sweep() {
  const int heads[][2] = {{1, 1}, {8, 8}, {32, 8}, {12, 4}, {6, 2}, {16, 1}, {28, 4}, {40, 8}};
  const int sqs[] = {0, 1, 5, 127, 128, 129, 256, 257, 512, 1000, 2048};
  const int skvs[] = {0, 1, 63, 64, 65, 700, 4096, 16384};
  const fa_dtype ods[] = {FA_BF16, FA_FP32};
  const int cus[] = {0, 256, 80, 1};
  const int splits[] = {0, 1, 3, 64};
  const int packs[] = {0, 1, 2, 4, 8};
  const int waves[] = {0, 4, 8};
  for (int c : cus) {
    set_env("FA_NUM_CUS", c);
    for (int f = 0; f < 4; ++f) {
      // override sets: none / splits / packs / waves
      const int nv = f == 0 ? 1 : f == 1 ? 4 : f == 2 ? 5 : 3;
      for (int vi = 0; vi < nv; ++vi) {
        set_env("FA_PREFILL_SPLITS", f == 1 ? splits[vi] : 0);
        set_env("FA_PREFILL_PACK", f == 2 ? packs[vi] : 0);
        set_env("FA_PREFILL_WAVES", f == 3 ? waves[vi] : 0);
        for (const auto& h : heads)
          for (int Sq : sqs)
            for (int Skv : skvs)
              for (int D : {64, 128}) {
                if (f > 0 && (Sq % 3 != 0 && Sq != 1)) continue;  // thinner override sweeps
                const int B = 1 + (Sq + Skv) % 3;
                const int causal = (Sq + Skv / 64) & 1;
                const fa_dtype od = ods[(Skv / 7 + Sq) & 1];
                prefill_case(B, h[0], h[1], Sq, Skv, D, causal, od, ((Sq ^ Skv) & 2) != 0);
              }
      }
    }
  }
  set_env("FA_NUM_CUS", 0);
  set_env("FA_PREFILL_SPLITS", 0);
  set_env("FA_PREFILL_PACK", 0);
  set_env("FA_PREFILL_WAVES", 0);
}

void decode_case(int B, int Sq, int Hq, int Hkv, fa_kv_layout layout, int page_size,
                 int max_seq_len, int num_splits) {
  const int Dqk = layout == FA_KV_MLA_SHARED ? 576 : 128;
  const int Dv = layout == FA_KV_MLA_SHARED ? 512 : 128;
  const size_t ws = Sq == 1 ? fa_decode_workspace_size(B, Hq, Hkv, Dqk, Dv, page_size,
                                                       max_seq_len, layout, num_splits)
                            : fa_decode_multi_workspace_size(B, Sq, Hq, Hkv, Dqk, Dv, page_size,
                                                             max_seq_len, layout, num_splits);
  Workspace w(ws);
  const int max_pages = std::max(1, (int)cdiv(max_seq_len, page_size));
  g_seen = Seen{};
  int rc;
  if (Sq == 1)
    rc = fa_decode_paged(fake(1), fake(2), (const int32_t*)fake(3), (const int32_t*)fake(4),
                         1000, fake(5), (float*)fake(6), B, Hq, Hkv, Dqk, Dv, page_size,
                         max_pages, max_seq_len, layout, 0.07f, num_splits, FA_BF16, w.p, ws,
                         nullptr);
  else
    rc = fa_decode_paged_multi(fake(1), fake(2), (const int32_t*)fake(3),
                               (const int32_t*)fake(4), 1000, fake(5), (float*)fake(6), B, Sq,
                               Hq, Hkv, Dqk, Dv, page_size, max_pages, max_seq_len, layout, 0.07f,
                               num_splits, FA_BF16, w.p, ws, nullptr);
  ++g_calls;
  CHECK(rc == FA_OK, "decode rc %d B%d Sq%d Hq%d Hkv%d layout%d page%d len%d splits%d", rc, B,
        Sq, Hq, Hkv, (int)layout, page_size, max_seq_len, num_splits);
  if (rc != FA_OK) return;
  const int launched = g_seen.dsplit + g_seen.dmla;
  CHECK(launched == (B > 0), "launches %d", launched);
  CHECK(g_seen.combine == (g_seen.splits > 1 ? 1 : 0), "combine");
  if (Sq == 1 && B > 0) {
    const int ns = fa_decode_num_splits(B, Hq, Hkv, Dqk, Dv, page_size, max_seq_len, layout,
                                        num_splits);
    CHECK(ns == g_seen.splits, "num_splits query %d, call %d", ns, g_seen.splits);
    // The entry point that allocates nothing runs the same plan in the static
    // scratch, or refuses it.
    g_seen = Seen{};
    g_touch = true;
    rc = fa_decode_paged_noalloc(fake(1), fake(2), (const int32_t*)fake(3),
                                 (const int32_t*)fake(4), 1000, fake(5), (float*)fake(6), B, Hq,
                                 Hkv, Dqk, Dv, page_size, max_pages, max_seq_len, layout, 0.07f,
                                 num_splits, FA_BF16, nullptr);
    ++g_calls;
    if (ws > fa::NOALLOC_SCRATCH_BYTES)
      CHECK(rc == FA_ERR_SCRATCH, "noalloc rc %d for %zu bytes", rc, ws);
    else
      CHECK(rc == FA_OK && g_seen.splits == ns, "noalloc rc %d splits %d", rc, g_seen.splits);
  }
}

void decode_sweep() {
  const int gqa[][2] = {{32, 8}, {8, 8}, {64, 8}, {16, 1}, {28, 4}};
  const int mla[] = {16, 32, 64, 128};
  const int lens[] = {0, 1, 31, 32, 33, 1000, 2048, 2049, 8192, 70000};
  const int pages[] = {1, 16, 5};
  const int nsp[] = {0, 1, 3, 100};
  const int cus[] = {0, 256, 40};
  for (int c : cus) {
    set_env("FA_NUM_CUS", c);
    for (int mh : {0, 32, 64}) {
      set_env("FA_MLA_HEADS", mh);
      for (int B : {0, 1, 4, 33, 128})
        for (int Sq : {1, 2, 4, 64})
          for (int len : lens)
            for (int ps : pages)
              for (int ns : nsp) {
                if (mh == 0)
                  for (const auto& h : gqa) decode_case(B, Sq, h[0], h[1], FA_KV_SPLIT, ps, len, ns);
                for (int hq : mla) decode_case(B, Sq, hq, 1, FA_KV_MLA_SHARED, ps, len, ns);
              }
    }
  }
  set_env("FA_NUM_CUS", 0);
  set_env("FA_MLA_HEADS", 0);
}

// Arguments the front end must refuse before anything is launched.
void error_paths() {
  g_seen = Seen{};
  auto pf = [](const void* q, int B, int Hq, int Hkv, int Sq, int D, fa_dtype in, fa_dtype out,
               void* ws, size_t wsb) {
    ++g_calls;
    return fa_prefill_ex(q, fake(2), fake(3), fake(5), nullptr, B, Hq, Hkv, Sq, 64, D, 1, 0.1f,
                         in, out, ws, wsb, nullptr);
  };
  CHECK(pf(fake(1), 0, 8, 8, 16, 128, FA_BF16, FA_BF16, nullptr, 0) == FA_ERR_SHAPE, "B=0");
  CHECK(pf(fake(1), 1, 8, 3, 16, 128, FA_BF16, FA_BF16, nullptr, 0) == FA_ERR_SHAPE, "Hq%%Hkv");
  CHECK(pf(fake(1), 1, 8, 8, 16, 96, FA_BF16, FA_BF16, nullptr, 0) == FA_ERR_UNSUPPORTED, "D");
  CHECK(pf(fake(1), 1, 8, 8, 16, 128, FA_FP32, FA_BF16, nullptr, 0) == FA_ERR_UNSUPPORTED, "in");
  CHECK(pf(nullptr, 1, 8, 8, 16, 128, FA_BF16, FA_BF16, nullptr, 0) == FA_ERR_NULL, "q null");
  CHECK(pf((char*)fake(1) + 8, 1, 8, 8, 16, 128, FA_BF16, FA_BF16, nullptr, 0) == FA_ERR_ALIGN,
        "q align");
  CHECK(pf(fake(1), 1, 8, 8, 16, 128, FA_BF16, FA_BF16, (char*)fake(7) + 4, 1 << 20) ==
            FA_ERR_ALIGN,
        "workspace align");
  setenv("FA_PREFILL_SPLITS", "4", 1);
  {
    ++g_calls;
    const size_t need = fa_prefill_workspace_size(1, 8, 8, 128, 4096, 128, 1, FA_BF16);
    Buf w(need);
    CHECK(need > 0 && fa_prefill_ex(fake(1), fake(2), fake(3), fake(5), nullptr, 1, 8, 8, 128,
                                    4096, 128, 1, 0.1f, FA_BF16, FA_BF16, w.p, need - 16,
                                    nullptr) == FA_ERR_WORKSPACE,
          "short workspace");
  }
  unsetenv("FA_PREFILL_SPLITS");
  // Masks: null, misaligned, strides.
  auto pm = [](const void* m, int64_t ms, int64_t mbs) {
    ++g_calls;
    return fa_prefill_mask(fake(1), fake(2), fake(3), m, ms, mbs, fake(5), nullptr, 1, 8, 8, 16,
                           100, 128, 0, 0.1f, FA_BF16, FA_BF16, nullptr, 0, nullptr);
  };
  CHECK(pm(nullptr, 104, 0) == FA_ERR_NULL, "mask null");
  CHECK(pm((char*)fake(4) + 8, 104, 0) == FA_ERR_ALIGN, "mask align");
  CHECK(pm(fake(4), 100, 0) == FA_ERR_ALIGN, "mask stride %% 8");
  CHECK(pm(fake(4), 96, 0) == FA_ERR_SHAPE, "mask stride < Skv");
  CHECK(pm(fake(4), 104, 12) == FA_ERR_ALIGN, "batch stride %% 8");
  // Decode.
  auto dc = [](int Sq, int Hq, int Hkv, int Dqk, int Dv, fa_kv_layout lay, int ps, int mp,
               int len, int np) {
    ++g_calls;
    return fa_decode_paged_multi(fake(1), fake(2), (const int32_t*)fake(3),
                                 (const int32_t*)fake(4), np, fake(5), nullptr, 2, Sq, Hq, Hkv,
                                 Dqk, Dv, ps, mp, len, lay, 0.1f, 0, FA_BF16, nullptr, 0, nullptr);
  };
  CHECK(dc(1, 32, 8, 128, 128, FA_KV_SPLIT, 16, 4, 64, 8) == FA_OK, "valid decode");
  CHECK(dc(0, 32, 8, 128, 128, FA_KV_SPLIT, 16, 4, 64, 8) == FA_ERR_SHAPE, "Sq=0");
  CHECK(dc(65, 32, 8, 128, 128, FA_KV_SPLIT, 16, 4, 64, 8) == FA_ERR_SHAPE, "Sq=65");
  CHECK(dc(1, 32, 8, 128, 128, FA_KV_SPLIT, 16, 3, 64, 8) == FA_ERR_SHAPE, "pages short");
  CHECK(dc(1, 32, 8, 128, 128, FA_KV_SPLIT, 16, 4, 64, 0) == FA_ERR_SHAPE, "no pages");
  CHECK(dc(1, 32, 8, 64, 64, FA_KV_SPLIT, 16, 4, 64, 8) == FA_ERR_UNSUPPORTED, "D=64 decode");
  CHECK(dc(1, 64, 64, 128, 128, FA_KV_SPLIT, 65536, 1, 64, 8) == FA_ERR_SHAPE, "2 GiB page");
  CHECK(dc(1, 64, 2, 576, 512, FA_KV_MLA_SHARED, 1, 64, 64, 8) == FA_ERR_SHAPE, "MLA Hkv=2");
  CHECK(dc(1, 64, 1, 512, 512, FA_KV_MLA_SHARED, 1, 64, 64, 8) == FA_ERR_UNSUPPORTED, "MLA D");
  CHECK(g_seen.combine == 0, "a refused call launched a combine");
  for (int s = 0; s >= -8; --s) CHECK(fa_strerror(s) && *fa_strerror(s), "strerror %d", s);
}

}  // namespace

int main(int argc, char** argv) {
  const std::string mode = argc > 1 ? argv[1] : "sweep";
  if (mode == "log") {
    Buf w(fa_prefill_workspace_size(1, 32, 8, 512, 16384, 128, 1, FA_BF16));
    fa_prefill_ex(fake(1), fake(2), fake(3), fake(5), nullptr, 1, 32, 8, 512, 16384, 128, 1,
                  0.088f, FA_BF16, FA_BF16, w.p,
                  fa_prefill_workspace_size(1, 32, 8, 512, 16384, 128, 1, FA_BF16), nullptr);
    fa_decode_paged(fake(1), fake(2), (const int32_t*)fake(3), (const int32_t*)fake(4), 1000,
                    fake(5), nullptr, 128, 64, 1, 576, 512, 1, 2048, 2048, FA_KV_MLA_SHARED,
                    0.07f, 0, FA_BF16, nullptr, 0, nullptr);
    std::printf("log mode done\n");
    return 0;
  }
  // The device query: the stubbed device reports g_stub_cus compute units,
  // and the planner must use them when FA_NUM_CUS is not set.
  unsetenv("FA_NUM_CUS");
  {
    const size_t a = fa_prefill_workspace_size(1, 32, 8, 512, 16384, 128, 1, FA_BF16);
    setenv("FA_NUM_CUS", std::to_string(g_stub_cus).c_str(), 1);
    const size_t b = fa_prefill_workspace_size(1, 32, 8, 512, 16384, 128, 1, FA_BF16);
    setenv("FA_NUM_CUS", "256", 1);
    const size_t c = fa_prefill_workspace_size(1, 32, 8, 512, 16384, 128, 1, FA_BF16);
    unsetenv("FA_NUM_CUS");
    CHECK(a == b, "device query %zu vs forced %zu", a, b);
    CHECK(c >= b, "more CUs planned fewer splits");
  }
  error_paths();
  prefill_sweep();
  decode_sweep();
  std::free(g_scratch);
  if (g_failures) {
    std::fprintf(stderr, "%d failures\n", g_failures);
    return 1;
  }
  std::printf("checked %ld calls\n", g_calls);
  return 0;
}
