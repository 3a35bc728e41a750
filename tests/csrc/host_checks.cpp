// Debug build of the library's host code, run on the CPU.  Compiled with QMOE_DEBUG_BOUNDS and
// the address and undefined-behaviour sanitizers on the host side, this program includes the
// library source itself (qmoe.hip, so the checks reach its internal functions) and runs the
// host logic and the index math that host and device share with every bounds assertion on:
//   - argument validation at and just past the limit of every dimension;
//   - the workspace layout: regions in order, 256-byte aligned and disjoint, each as large as
//     what its users index, for every configured shape, the limit shapes and many token
//     counts; the one-token hand-off areas (asserted where their pointers are made) and LDS map;
//   - the store's chunk map: every chunk of a block packed and unpacked on the host with
//     exactly sized buffers, every 16-byte chunk of the block produced once, every canonical
//     code, scale and bias consumed once, and the round trip exact;
//   - bucketing: the scan word's fields at the largest call, the block-count bound and the
//     block table (every row of every expert in exactly one block) for skewed, flat and
//     random count vectors, and the LDS the bucketing launch asks for;
//   - the expert cache policy's invariants over random call streams, and its refusals.
// Prints "host checks: ok" and exits 0, or aborts at the first failed check.
#include "qmoe.hip"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

namespace {

long n_checks = 0;
#define CHECK(c)                                                                        \
  do {                                                                                  \
    ++n_checks;                                                                         \
    if (!(c)) {                                                                         \
      std::fprintf(stderr, "host check failed: %s (%s:%d)\n", #c, __FILE__, __LINE__); \
      std::abort();                                                                     \
    }                                                                                   \
  } while (0)

struct Shape {
  const char *name;
  int H, E, k, I, Is, bits;
};

// the configured workloads' layer shapes, the smallest and largest accepted ones, and a few
// with no power-of-two dimension
const Shape SHAPES[] = {
    {"tiny", 256, 16, 2, 128, 128, 4},
    {"tiny_int8", 256, 16, 2, 128, 128, 8},
    {"gemma4_26b_a4b", 2816, 128, 8, 704, 2112, 4},
    {"gemma4_26b_a4b_int8", 2816, 128, 8, 704, 2112, 8},
    {"qwen3_next_80b_a3b", 2048, 512, 10, 512, 512, 4},
    {"qwen3_6_35b_a3b", 2048, 256, 8, 512, 512, 4},
    {"smallest", 64, 1, 1, 64, 0, 4},
    {"odd", 192, 33, 3, 192, 320, 4},
    {"odd_int8", 320, 7, 7, 448, 0, 8},
    {"widest", 8192, 1024, 32, 4096, 4096, 4},
    {"widest_int8", 8192, 1024, 32, 4096, 4096, 8},
};

qmoe_dims dims_of(const Shape &s) {
  qmoe_dims d;
  std::memset(&d, 0, sizeof d);
  d.hidden = s.H;
  d.n_experts = s.E;
  d.top_k = s.k;
  d.inter = s.I;
  d.shared_inter = s.Is;
  d.group = GROUP;
  d.expert_bits = s.bits;
  return d;
}

// A pointer the host code only offsets and compares, never dereferences.
template <class T>
T *fake(uintptr_t a) { return reinterpret_cast<T *>(a); }

// ---------------------------------------------------------------- validation
void check_validation() {
  const qmoe_dims d = dims_of(SHAPES[2]);
  CHECK(check_dims(&d) == QMOE_OK);
  CHECK(check_dims(nullptr) == QMOE_ERR_ARG);
  struct Case {
    int field, value;
    bool ok;
  };
  // field: 0 hidden, 1 inter, 2 shared_inter, 3 n_experts, 4 top_k, 5 expert_bits, 6 group
  const Case cases[] = {
      {0, 64, true},    {0, 8192, true},  {0, 8256, false}, {0, 0, false},   {0, -64, false},
      {0, 100, false},  {1, 64, true},    {1, 4096, true},  {1, 4160, false}, {1, 96, false},
      {2, 0, true},     {2, 4096, true},  {2, 4160, false}, {2, 32, false},  {3, 8, true},
      {3, 1024, true},  {3, 1025, false}, {3, 0, false},    {3, 7, false},   {4, 1, true},
      {4, 32, true},    {4, 33, false},   {4, 0, false},    {4, 8, true},     {5, 0, true},    {5, 4, true},
      {5, 8, true},     {5, 2, false},    {5, 16, false},   {6, 32, false},  {6, 128, false},
      {4, -1, false},
  };
  for (const Case &c : cases) {
    qmoe_dims e = d;   // E = 128, k = 8
    int *f[] = {&e.hidden, &e.inter, &e.shared_inter, &e.n_experts, &e.top_k, &e.expert_bits,
                &e.group};
    *f[c.field] = c.value;
    CHECK((check_dims(&e) == QMOE_OK) == c.ok);
  }
  {
    qmoe_dims e = dims_of(SHAPES[9]);   // E = 1024: top_k 32 is the limit
    CHECK(check_dims(&e) == QMOE_OK);
    e.top_k = 33;
    CHECK(check_dims(&e) == QMOE_ERR_SHAPE);
  }
  CHECK(check_T(-1) == QMOE_ERR_SHAPE);
  CHECK(check_T(0) == QMOE_OK);
  CHECK(check_T(MAX_T) == QMOE_OK);
  CHECK(check_T(MAX_T + 1) == QMOE_ERR_SHAPE);
  const size_t need = ws_layout(&d, 128).total;
  CHECK(check_ws(&d, 128, fake<void>(0x100000), need) == QMOE_OK);
  CHECK(check_ws(&d, 128, fake<void>(0x100000), need - 1) == QMOE_ERR_WORKSPACE);
  CHECK(check_ws(&d, 128, fake<void>(0x100010), need) == QMOE_ERR_WORKSPACE);
  CHECK(check_ws(&d, 128, nullptr, need) == QMOE_ERR_WORKSPACE);

  qmoe_layer L;
  std::memset(&L, 0, sizeof L);
  L.d = d;
  L.r.codes = fake<uint8_t>(0x200000);
  L.r.scales = fake<uint16_t>(0x300000);
  L.r.biases = fake<uint16_t>(0x400000);
  L.r.per_expert_scale = fake<float>(0x500000);
  L.experts = fake<void>(0x1000000);
  L.expert_stride = block_stride_bytes(d.hidden, d.inter, kshift_of(&d));
  CHECK(check_layer(&L) == QMOE_OK);
  qmoe_layer M = L;
  M.expert_stride -= 256;
  CHECK(check_layer(&M) == QMOE_ERR_ARG);
  M = L;
  M.experts = fake<void>(0x1000080);
  CHECK(check_layer(&M) == QMOE_ERR_ARG);
  M = L;
  M.d.shared_inter = 0;
  M.shared = fake<void>(0x2000000);
  CHECK(check_layer(&M) == QMOE_ERR_ARG);
  M = L;
  M.r.codes = fake<uint8_t>(0x200004);
  CHECK(check_layer(&M) == QMOE_ERR_ARG);
  M = L;
  M.r.scales = nullptr;
  CHECK(check_layer(&M) == QMOE_ERR_ARG);
}

// ---------------------------------------------------------------- workspace layout
void check_layout(const Shape &s, int T) {
  const qmoe_dims d = dims_of(s);
  if (check_dims(&d) != QMOE_OK) return;
  const WsLayout w = ws_layout(&d, T);
  size_t o = 0;
  for (int i = 0; i < w.n_reg; ++i) {
    CHECK(w.reg[i].off == o && o % 256 == 0);
    o += w.reg[i].bytes;
  }
  CHECK(o == w.total);
  const size_t Tz = (size_t)T, Tc = std::min<size_t>(Tz, CHUNK_TOKENS), k = s.k, E = s.E,
               H = s.H, I = s.I, Is = s.Is;
  // bytes each region's users index for a call of T tokens (multi-token calls run chunk by
  // chunk: the per-chunk regions hold one chunk)
  const struct {
    size_t off, need;
  } needs[] = {
      {w.logits, Tz * E * 4},          {w.tidx, Tz * k * 4},
      {w.tw, Tz * k * 4},              {w.counts, E * 4},
      {w.offsets, (E + 1) * 4},        {w.sorted, Tc * k * 4},
      {w.active, E * 4},               {w.nact, 4},
      {w.slot_tab, (size_t)bucket_max_blocks((int)(Tc * k), (int)E) * 16},
      {w.slot_ids, Tc * k * 4},        {w.hr_hi, Tz * k * I * 2},
      {w.hr_lo, Tz * k * I * 2},       {w.hs_hi, Tz * Is * 2},
      {w.hs_lo, Tz * Is * 2},          {w.y, Tc * k * H * 4},
      {w.ysh, Tc * H * 4},             {w.gx, Tz * (H / GROUP) * 4},
      {w.ghr, Tz * k * (I / GROUP) * 4}, {w.ghs, Tz * (Is / GROUP) * 4},
      {w.rpart, (size_t)rmf_splits((int)H) * Tc * E * 4},
      {w.rss, (size_t)rmf_splits((int)H) * Tc * 4},
  };
  for (const auto &n : needs) {
    if (n.need > w.bytes_at(n.off))
      std::fprintf(stderr, "%s T=%d: region at %zu holds %zu bytes, %zu indexed\n", s.name, T, n.off,
                   w.bytes_at(n.off), n.need);
    CHECK(n.need <= w.bytes_at(n.off));
  }
  // the one-token areas sit where a one-token layout puts them, whatever T the workspace was
  // sized for
  const WsLayout w1 = ws_layout(&d, 1);
  CHECK(w.dec_logits == w1.dec_logits && w.dec_hr == w1.dec_hr && w.dec_hsh == w1.dec_hsh &&
        w.dec_yr == w1.dec_yr && w.dec_ysh == w1.dec_ysh && w.dec_nrm == w1.dec_nrm &&
        w.dec_tk == w1.dec_tk && w.dec_x == w1.dec_x && w.dec_tab == w1.dec_tab);
}

void check_decode_setup(const Shape &s) {
  const qmoe_dims d = dims_of(s);
  if (check_dims(&d) != QMOE_OK || !decode_fits(&d)) return;
  for (int with_shared = 0; with_shared < 2; ++with_shared) {
    if (with_shared && s.Is == 0) continue;
    qmoe_layer L;
    std::memset(&L, 0, sizeof L);
    L.d = d;
    L.experts = fake<void>(0x1000000);
    L.expert_stride = block_stride_bytes(d.hidden, d.inter, kshift_of(&d));
    if (with_shared) L.shared = fake<void>(0x2000000);
    for (int T : {1, 128}) {
      const WsLayout wl = ws_layout(&d, T);
      // asserts every hand-off area's copies inside its region and the LDS map inside the LDS
      const DecodeArgs a = make_decode_args(&L, fake<uint16_t>(0x10000), fake<uint16_t>(0x20000),
                                            nullptr, fake<int32_t>(0x30000),
                                            fake<float>(0x40000), fake<void>(0x100000), wl);
      CHECK(a.nRD > 0 && a.nRG == s.k * (s.I / 16));
      const DecLds lds = dec_lds_of(&d, with_shared != 0);
      const size_t regions[] = {lds.tk, lds.tks, lds.pes, lds.red, lds.nrm, lds.xw, lds.x, lds.xs};
      for (int i = 1; i < 8; ++i) CHECK(regions[i] > regions[i - 1]);
      CHECK(lds.hf == lds.x && lds.hh > lds.hf && lds.hl > lds.hh && lds.hs > lds.hl &&
            lds.comb > lds.hs && lds.total <= 160 * 1024);
    }
  }
}

// ---------------------------------------------------------------- store chunk map
void check_store(const Shape &s, std::mt19937_64 &rng) {
  const int H = s.H, I = s.I, kshift = s.bits == 8 ? 1 : 0;
  const BlockGeom g = block_geom(H, I, kshift);
  const long n = ((long)g.gu_tiles * g.gu_ks + (long)g.d_tiles * g.d_ks) * 64;
  const size_t code_gu = (size_t)I * (kshift ? H : H / 2), code_d = (size_t)H * (kshift ? I : I / 2);
  const size_t grp_gu = (size_t)I * (H / GROUP), grp_d = (size_t)H * (I / GROUP);
  // canonical arrays, exactly sized (the sanitizer sees any access past them)
  std::vector<uint8_t> gq(code_gu), uq(code_gu), dq(code_d);
  std::vector<uint16_t> gs(grp_gu), gb(grp_gu), us(grp_gu), ub(grp_gu), ds(grp_d), db(grp_d);
  for (auto *v : {&gq, &uq, &dq})
    for (auto &b : *v) b = (uint8_t)rng();
  // scales: normal bf16 values (16 s stays exact for the 8-bit split); biases: any bits
  auto bf16_normal = [&]() { return (uint16_t)(0x3800u + (rng() % 0x1000u) + ((rng() & 1) << 15)); };
  for (auto *v : {&gs, &us, &ds})
    for (auto &x : *v) x = bf16_normal();
  for (auto *v : {&gb, &ub, &db})
    for (auto &x : *v) x = (uint16_t)rng();
  const CanonExpert c{gq.data(), uq.data(), dq.data(), gs.data(), gb.data(),
                      us.data(), ub.data(), ds.data(), db.data()};
  const size_t block_bytes = g.gu_bytes + g.d_bytes;
  CHECK(block_bytes <= block_stride_bytes(H, I, kshift));

  // the chunk map is one to one onto the block's chunks and onto the canonical elements
  std::vector<uint8_t> chunk_seen(block_bytes / 16, 0);
  std::vector<uint8_t> code_seen_g(code_gu * 2, 0), code_seen_u(code_gu * 2, 0), code_seen_d(code_d * 2, 0);
  for (long id = 0; id < n; ++id) {
    ChunkPos p;
    CHECK(chunk_pos(id, H, I, kshift, p));
    CHECK(p.rr >= 0 && p.rr < 32 && p.half >= 0 && p.half < 2 && p.ks >= 0);
    CHECK(p.row >= 0 && p.row < (p.gu ? I : H) && p.group >= 0 && p.group < p.K / GROUP);
    const size_t off = (p.gu ? 0 : g.gu_bytes) + (size_t)p.kst * KSTEP_BYTES + p.chunk * 16;
    CHECK(off + 16 <= (p.gu ? g.gu_bytes : block_bytes));
    CHECK(chunk_seen[off / 16]++ == 0);
    std::vector<uint8_t> &seen = p.gu ? (p.rr >= 16 ? code_seen_u : code_seen_g) : code_seen_d;
    for (int j = 0; j < 32; ++j) {
      const size_t el = (size_t)p.row * p.K + p.group * GROUP + p.half * 32 + j;
      const size_t slot = kshift ? el * 2 + p.plane : el;   // 8-bit: each code in two planes
      CHECK(slot < seen.size() && seen[slot]++ == 0);
    }
  }
  {
    ChunkPos p;
    CHECK(!chunk_pos(n, H, I, kshift, p) && !chunk_pos(-1, H, I, kshift, p));
  }
  const size_t per_code = kshift ? 2 : 1;   // element slots per canonical element
  const size_t els_gu = (size_t)I * H, els_d = (size_t)H * I;
  CHECK((size_t)std::count(code_seen_g.begin(), code_seen_g.begin() + els_gu * per_code, 1) == els_gu * per_code);
  CHECK((size_t)std::count(code_seen_u.begin(), code_seen_u.begin() + els_gu * per_code, 1) == els_gu * per_code);
  CHECK((size_t)std::count(code_seen_d.begin(), code_seen_d.begin() + els_d * per_code, 1) == els_d * per_code);
  // every 16-byte chunk of the block is either a code chunk or part of a scale|bias area
  for (size_t i = 0; i < chunk_seen.size(); ++i) {
    const size_t in_step = (i * 16 - (i * 16 >= g.gu_bytes ? g.gu_bytes : 0)) % KSTEP_BYTES;
    CHECK(chunk_seen[i] == (in_step < 1024 ? 1 : 0));
  }

  // pack twice over different fills: every byte of the block is written (both runs agree)
  std::vector<uint8_t> blk_a(block_bytes, 0x00), blk_b(block_bytes, 0xFF);
  for (long id = 0; id < n + 300; ++id) {   // ids past the end are no-ops
    pack_chunk(c, H, I, kshift, blk_a.data(), id);
    pack_chunk(c, H, I, kshift, blk_b.data(), id);
  }
  CHECK(blk_a == blk_b);

  // unpack into sentinel-filled arrays: every canonical byte and word comes back
  std::vector<uint8_t> gq2(code_gu, 0x5A), uq2(code_gu, 0x5A), dq2(code_d, 0x5A);
  std::vector<uint16_t> gs2(grp_gu, 0xA5A5), gb2(grp_gu, 0xA5A5), us2(grp_gu, 0xA5A5),
      ub2(grp_gu, 0xA5A5), ds2(grp_d, 0xA5A5), db2(grp_d, 0xA5A5);
  const CanonExpertOut co{gq2.data(), uq2.data(), dq2.data(), gs2.data(), gb2.data(),
                          us2.data(), ub2.data(), ds2.data(), db2.data()};
  for (long id = 0; id < n + 300; ++id) unpack_chunk(blk_a.data(), H, I, kshift, co, id);
  CHECK(gq2 == gq && uq2 == uq && dq2 == dq);
  CHECK(gs2 == gs && gb2 == gb && us2 == us && ub2 == ub && ds2 == ds && db2 == db);
}

// ---------------------------------------------------------------- bucketing
void check_bucket_counts(const std::vector<int> &cnt) {
  const int E = (int)cnt.size();
  long long scan = 0;
  long N = 0, blocks = 0, active = 0;
  for (int c : cnt) {
    scan += bucket_scan_word(c);
    N += c;
    blocks += (c + BUCKET_BLOCK_ROWS - 1) / BUCKET_BLOCK_ROWS;
    active += c > 0;
  }
  CHECK(N <= BUCKET_MAX_N);
  CHECK(bucket_scan_rows(scan) == N && bucket_scan_blocks(scan) == blocks &&
        bucket_scan_flags(scan) == active);
  const int nmax = bucket_max_blocks((int)N, E);
  CHECK(blocks <= nmax);
  // the block table as the bucketing kernel writes it: every row of every expert in exactly
  // one block, blocks in expert order, at most BUCKET_BLOCK_ROWS rows each
  long pos = 0, b_all = 0;
  for (int e = 0; e < E; ++e) {
    const int c = cnt[e];
    long covered = 0;
    for (int b = 0; b * BUCKET_BLOCK_ROWS < c; ++b, ++b_all) {
      const qmoe_u32x4 t = bucket_block_entry(e, c, (int)pos, 1000 + e, b);
      CHECK((int)t.x == e && (long)t.y == pos + covered && t.z >= 1 && t.z <= BUCKET_BLOCK_ROWS);
      CHECK(t.w == (b == 0 ? 1000u + e : 0xFFFFFFFFu));
      covered += t.z;
    }
    CHECK(covered == c);
    pos += c;
  }
  CHECK(b_all == blocks && pos == N);
}

void check_bucket(std::mt19937_64 &rng) {
  for (int E : {1, 2, 7, 16, 128, 256, 512, 1024}) {
    for (long N : {0L, 1L, 15L, 16L, 17L, 1000L, 4096L, (long)BUCKET_MAX_N}) {
      std::vector<int> cnt(E, 0);
      cnt[0] = (int)N;                             // every assignment on one expert
      check_bucket_counts(cnt);
      std::fill(cnt.begin(), cnt.end(), 0);        // 17 rows per expert (two blocks each)
      for (long left = N, e = 0; left > 0; e = (e + 1) % E) {
        const int add = (int)std::min<long>(left, 17);
        cnt[e] += add;
        left -= add;
      }
      check_bucket_counts(cnt);
      std::fill(cnt.begin(), cnt.end(), 0);        // one row each, the rest on the last
      for (long i = 0; i < N; ++i) ++cnt[i < E ? i : E - 1];
      check_bucket_counts(cnt);
      std::fill(cnt.begin(), cnt.end(), 0);        // random
      for (long i = 0; i < std::min<long>(N, 20000); ++i) ++cnt[rng() % E];
      if (N > 20000) cnt[rng() % E] += (int)(N - 20000);
      check_bucket_counts(cnt);
    }
  }
  // the LDS of the bucketing launch, for every call the layer and bucketing entries make
  for (int E = 1; E <= MAX_EXPERTS; E += (E < 64 ? 1 : 31))
    for (int N = 0; N <= 8192; N += (N < 256 ? 1 : 61)) {
      CHECK(bucket_lds_bytes(N, E) <= 160 * 1024);
      CHECK(bucket_max_blocks(N, E) >= 0);
    }
}

// ---------------------------------------------------------------- cache policy
void check_cache(std::mt19937_64 &rng) {
  for (auto [E, S] : {std::pair<int, int>{128, 16}, {512, 40}, {16, 16}, {8, 1}}) {
    ExpertCachePolicy pol(E, S);
    CachePlan p;
    // Zipf-like ids: expert e with weight 1 / (e + 1)
    std::vector<double> cdf(E);
    double acc = 0;
    for (int e = 0; e < E; ++e) cdf[e] = (acc += 1.0 / (e + 1));
    for (int call = 0; call < 4000; ++call) {
      const int n = 1 + (int)(rng() % std::min(S, 24));
      std::vector<int32_t> ids(n);
      for (auto &id : ids) {
        const double u = std::uniform_real_distribution<double>(0, acc)(rng);
        id = (int32_t)(std::lower_bound(cdf.begin(), cdf.end(), u) - cdf.begin());
        if (id >= E) id = E - 1;
      }
      std::vector<int32_t> uniq(ids);
      std::sort(uniq.begin(), uniq.end());
      const int distinct = (int)(std::unique(uniq.begin(), uniq.end()) - uniq.begin());
      const int64_t h0 = pol.hits(), m0 = pol.misses();
      const bool ok_call = pol.plan(ids.data(), n, p);   // asserts the invariants inside
      CHECK(ok_call == (distinct <= S));
      if (ok_call) CHECK(pol.hits() - h0 + pol.misses() - m0 == distinct);
      else CHECK(pol.hits() == h0 && pol.misses() == m0);
    }
    std::vector<int32_t> bad = {0, E};
    const int64_t h0 = pol.hits(), m0 = pol.misses();
    CHECK(!pol.plan(bad.data(), 2, p) && pol.hits() == h0 && pol.misses() == m0);
    bad = {-1};
    CHECK(!pol.plan(bad.data(), 1, p));
  }
}

}  // namespace

int main() {
  std::mt19937_64 rng(20261203);
  check_validation();
  for (const Shape &s : SHAPES) {
    for (int T : {0, 1, 2, 15, 16, 17, 127, 128, 129, 1000, 10240, MAX_T}) check_layout(s, T);
    check_decode_setup(s);
  }
  for (const Shape &s : SHAPES)
    if (s.H * (size_t)s.I <= 2816 * 704) check_store(s, rng);   // every shape up to Gemma's
  check_bucket(rng);
  check_cache(rng);
  std::printf("host checks: ok (%ld checks)\n", n_checks);
  return 0;
}
