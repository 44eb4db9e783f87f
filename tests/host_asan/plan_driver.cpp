// Host-only driver of the planner for a sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer, g++): plans random iterations and the pages' workload shapes,
// including the 128K-context metadata of 524,288 block-table entries, and checks every
// plan's work lists: each visible (row, query head, position) is scored exactly once, by
// an MFMA tile or a split-KV item, and every partial slot an output uses is distinct and
// inside its combine row.  Invalid metadata must be refused with the right status.
//
// The planner's three device hooks are replaced by host stubs below (the plans are built
// with VA_FLAG_HOST_ONLY, so no device buffer is made).  Exit status 0 = all checks passed.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <numeric>
#include <random>
#include <string>
#include <vector>

#include "va_internal.h"

namespace va {
va_status upload_plan(va_plan*) { return fail(VA_ERR_UNSUPPORTED, "host-only build: no device"); }
int device_compute_units() { return 0; }
void free_plan_device(va_plan* plan) { plan->dev = nullptr; }
bool prefill_kernel_available(const va_params& p) {
  return (p.dtype == VA_DTYPE_BF16 || p.dtype == VA_DTYPE_FP8_E4M3) && (p.head_dim == 64 || p.head_dim == 128);
}
}  // namespace va

namespace {

int g_failures = 0;
#define CHECK(cond, ...)                                      \
  do {                                                        \
    if (!(cond)) {                                            \
      std::fprintf(stderr, "CHECK failed (%s): ", #cond);     \
      std::fprintf(stderr, __VA_ARGS__);                      \
      std::fprintf(stderr, "\n");                             \
      if (++g_failures > 20) std::exit(1);                    \
    }                                                         \
  } while (0)

struct Case {
  std::string name;
  va_params p{};
  std::vector<int32_t> qs, qe, kv, bt;
};

template <typename T>
std::vector<T> exported(const va_plan* plan, int which) {
  const int32_t* data = nullptr;
  int64_t n = 0;
  int32_t w = 0;
  const va_status s = varlen_attn_plan_export(plan, which, &data, &n, &w);
  CHECK(s == VA_OK, "export %d: %s", which, varlen_attn_last_error());
  CHECK(n == 0 || size_t(w) * 4 == sizeof(T), "export %d: %d ints per entry", which, w);
  std::vector<T> out(static_cast<size_t>(n));
  if (n) std::copy_n(reinterpret_cast<const T*>(data), size_t(n), out.begin());
  return out;
}

// Checks the plan's work lists against the metadata; returns the number of outputs covered.
int64_t check_plan(const Case& c, const va_plan* plan) {
  const va_params& p = c.p;
  const int R = int(c.kv.size()), Hq = p.num_q_heads, g = p.num_q_heads / p.num_kv_heads;
  const int ps = p.page_size, stride = p.max_pages_per_req;
  va_plan_stats st{};
  CHECK(varlen_attn_plan_stats(plan, &st) == VA_OK, "%s: stats", c.name.c_str());
  const auto items = exported<va::SplitItem>(plan, 0);
  const auto cols = exported<va::Column>(plan, 1);
  const auto comb = exported<va::CombineRow>(plan, 2);
  const auto tiles = exported<va::PrefillTile>(plan, 3);
  const auto listed = exported<va::PrefillTile>(plan, 4);
  int64_t rows = 0;
  for (int r = 0; r < R; ++r) rows = std::max<int64_t>(rows, c.qe[r] > c.qs[r] ? c.qe[r] : 0);
  CHECK(st.total_q_rows == rows, "%s: total_q_rows", c.name.c_str());
  std::vector<int32_t> req_of_row(size_t(rows), -1);
  for (int r = 0; r < R; ++r)
    for (int t = c.qs[r]; t < c.qe[r]; ++t) req_of_row[size_t(t)] = r;
  auto key = [&](int row, int head) { return int64_t(row) * Hq + head; };
  std::map<int64_t, std::vector<std::pair<int, int>>> cover;   // output -> [k0, k1) intervals
  std::map<int64_t, std::vector<int>> slots;                   // output -> partial slots used
  std::map<int64_t, std::pair<int, int>> comb_of;              // output -> (pbase, nparts)
  std::map<int64_t, int> direct;
  for (const auto& cr : comb) {
    CHECK(cr.nparts >= 1 && cr.pbase >= 0 && int64_t(cr.pbase) + cr.nparts <= st.partial_slots, "%s: combine row",
          c.name.c_str());
    CHECK(comb_of.emplace(key(cr.q_row, cr.q_head), std::make_pair(cr.pbase, cr.nparts)).second,
          "%s: output combined twice", c.name.c_str());
  }
  auto same_pages = [&](int req, int r, int k0, int hi) {
    for (int j = k0 / ps; j <= (hi - 1) / ps; ++j)
      if (c.bt[size_t(req) * stride + j] != c.bt[size_t(r) * stride + j]) return false;
    return true;
  };
  auto col_ok = [&](const va::Column& col, int kvh) {
    if (col.q_row < 0 || col.q_row >= rows) return -1;
    const int r = req_of_row[size_t(col.q_row)];
    if (r < 0 || col.q_head / g != kvh) return -1;
    const int m = c.qe[r] - c.qs[r];
    return col.limit == c.kv[r] - m + (col.q_row - c.qs[r]) ? r : -1;
  };
  for (const auto& it : items) {
    CHECK(it.ncols >= 1 && it.ncols <= 32 && it.k0 < it.k1 && it.k0 % 16 == 0, "%s: item shape", c.name.c_str());
    CHECK(it.col0 >= 0 && size_t(it.col0) + it.ncols <= cols.size(), "%s: item columns", c.name.c_str());
    for (int i = 0; i < it.ncols; ++i) {
      const va::Column& col = cols[size_t(it.col0 + i)];
      const int r = col_ok(col, it.kvh);
      CHECK(r >= 0, "%s: item column", c.name.c_str());
      if (r < 0) continue;
      const int hi = std::min(it.k1, col.limit + 1);
      const int64_t o = key(col.q_row, col.q_head);
      if (hi > it.k0) {
        CHECK(same_pages(it.req, r, it.k0, hi), "%s: item reads another request's pages", c.name.c_str());
        cover[o].push_back({it.k0, hi});
      }
      if (it.flags & va::kItemDirect) {
        CHECK(!comb_of.count(o) && col.pbase == -1, "%s: direct item of a combined output", c.name.c_str());
        ++direct[o];
      } else {
        const auto cb = comb_of.find(o);
        CHECK(cb != comb_of.end() && cb->second.first == col.pbase && it.slot >= 0 && it.slot < cb->second.second,
              "%s: item slot", c.name.c_str());
        slots[o].push_back(it.slot);
      }
      if (!(it.flags & va::kItemMasked)) CHECK(it.k1 - 1 <= col.limit, "%s: unmasked item", c.name.c_str());
    }
  }
  int64_t n_list = 0;
  for (const auto& t : tiles) {
    CHECK(t.ncols >= 1 && t.ncols <= va::kPrefillCols && t.kbeg < t.kv_end, "%s: tile shape", c.name.c_str());
    if (t.flags & va::kTileColumnList) {
      ++n_list;
      CHECK(t.kbeg == t.S0 && t.pbase == -1, "%s: column-list tile", c.name.c_str());
      CHECK(t.c0 >= 0 && size_t(t.c0) + t.ncols <= cols.size(), "%s: tile columns", c.name.c_str());
      for (int i = 0; i < t.ncols; ++i) {
        const va::Column& col = cols[size_t(t.c0 + i)];
        const int r = col_ok(col, t.kvh);
        CHECK(r >= 0 && t.kbeg <= col.limit, "%s: column-list column", c.name.c_str());
        if (r < 0) continue;
        const int hi = std::min(t.kv_end, col.limit + 1);
        CHECK(same_pages(t.req, r, t.kbeg, hi), "%s: tile reads another request's pages", c.name.c_str());
        const int64_t o = key(col.q_row, col.q_head);
        cover[o].push_back({t.kbeg, hi});
        const auto cb = comb_of.find(o);
        CHECK(cb != comb_of.end() && cb->second.first == col.pbase && t.q0 >= 0 && t.q0 < cb->second.second,
              "%s: column-list slot", c.name.c_str());
        slots[o].push_back(t.q0);
      }
      continue;
    }
    const int r = t.req;
    CHECK(r >= 0 && r < R && t.q0 == c.qs[r] && t.S0 == c.kv[r] - (c.qe[r] - c.qs[r]), "%s: tile request",
          c.name.c_str());
    for (int col = t.c0; col < t.c0 + t.ncols; ++col) {
      const int row = t.q0 + col / g, head = t.kvh * g + col % g, limit = t.S0 + col / g;
      CHECK(row < c.qe[r], "%s: tile row past the request", c.name.c_str());
      const int hi = std::min(t.kv_end, limit + 1);
      CHECK(hi > t.kbeg, "%s: tile column sees no key", c.name.c_str());
      const int64_t o = key(row, head);
      cover[o].push_back({t.kbeg, hi});
      if (t.pbase >= 0) {
        const int slot = t.pbase + (col - t.c0) * t.pstride;
        const auto cb = comb_of.find(o);
        CHECK(cb != comb_of.end() && slot >= cb->second.first && slot < cb->second.first + cb->second.second,
              "%s: tile slot", c.name.c_str());
        slots[o].push_back(slot - (cb != comb_of.end() ? cb->second.first : 0));
      } else {
        CHECK(!comb_of.count(o), "%s: whole tile of a combined output", c.name.c_str());
        ++direct[o];
      }
    }
  }
  CHECK(int64_t(listed.size()) == n_list, "%s: column-list copies", c.name.c_str());
  for (const auto& d : direct) CHECK(d.second == 1 && !slots.count(d.first), "%s: direct output", c.name.c_str());
  for (auto& s : slots) {
    std::sort(s.second.begin(), s.second.end());
    CHECK(std::adjacent_find(s.second.begin(), s.second.end()) == s.second.end(), "%s: slot used twice",
          c.name.c_str());
    CHECK(int(s.second.size()) == comb_of[s.first].second, "%s: parts != nparts", c.name.c_str());
  }
  // every visible key of every output exactly once
  int64_t outputs = 0;
  for (int r = 0; r < R; ++r) {
    const int m = c.qe[r] - c.qs[r], S0 = c.kv[r] - m;
    for (int i = 0; i < m; ++i)
      for (int h = 0; h < Hq; ++h) {
        auto& iv = cover[key(c.qs[r] + i, h)];
        std::sort(iv.begin(), iv.end());
        int at = 0;
        bool ok = !iv.empty();
        for (const auto& x : iv) {
          ok = ok && x.first == at && x.second > x.first;
          at = x.second;
        }
        CHECK(ok && at == S0 + i + 1, "%s: request %d row %d head %d not covered exactly once", c.name.c_str(), r, i,
              h);
        ++outputs;
      }
  }
  int64_t nslots = 0;
  for (const auto& cb : comb_of) nslots += cb.second.second;
  CHECK(nslots == st.partial_slots, "%s: partial slots", c.name.c_str());
  std::vector<int64_t> loc(size_t(std::max<int64_t>(rows, 1)));
  CHECK(varlen_attn_plan_slots(plan, loc.data()) == VA_OK, "%s: slots", c.name.c_str());
  return outputs;
}

Case make(const std::string& name, const std::vector<int>& q_rows, const std::vector<int>& kvl, int hq, int hkv, int d,
          int ps, int dtype, std::mt19937_64& rng, int shared_pages = 0, int gap = 0) {
  Case c;
  c.name = name;
  const int R = int(kvl.size());
  int maxp = 1;
  for (int k : kvl) maxp = std::max(maxp, (k + ps - 1) / ps);
  int pages = shared_pages;
  for (int k : kvl) pages += (k + ps - 1) / ps - shared_pages;
  std::vector<int32_t> perm(size_t(std::max(pages, 1)));
  std::iota(perm.begin(), perm.end(), 0);
  std::shuffle(perm.begin(), perm.end(), rng);
  c.bt.assign(size_t(R) * maxp, -1);
  int next = shared_pages, row = 0;
  for (int r = 0; r < R; ++r) {
    const int np = (kvl[r] + ps - 1) / ps;
    for (int j = 0; j < np; ++j) c.bt[size_t(r) * maxp + j] = perm[size_t(j < shared_pages ? j : next++)];
    c.qs.push_back(row);
    row += q_rows[r];
    c.qe.push_back(row);
    row += gap;
    c.kv.push_back(kvl[r]);
  }
  c.p.num_q_heads = hq;
  c.p.num_kv_heads = hkv;
  c.p.head_dim = d;
  c.p.page_size = ps;
  c.p.num_pages = std::max(pages, 1);
  c.p.max_pages_per_req = maxp;
  c.p.dtype = dtype;
  c.p.flags = VA_FLAG_HOST_ONLY;
  return c;
}

int64_t run_case(const Case& c) {
  va_plan* plan = nullptr;
  size_t ws = 0;
  const va_status s = varlen_attn_plan(&c.p, int32_t(c.kv.size()), c.qs.data(), c.qe.data(), c.kv.data(),
                                       c.bt.data(), &plan, &ws);
  CHECK(s == VA_OK, "%s: plan failed: %s", c.name.c_str(), varlen_attn_last_error());
  if (s != VA_OK) return 0;
  const int64_t n = check_plan(c, plan);
  varlen_attn_plan_destroy(plan);
  return n;
}

void expect_refused(const Case& c, va_status want) {
  va_plan* plan = reinterpret_cast<va_plan*>(1);
  const va_status s = varlen_attn_plan(&c.p, int32_t(c.kv.size()), c.qs.empty() ? nullptr : c.qs.data(),
                                       c.qe.empty() ? nullptr : c.qe.data(), c.kv.empty() ? nullptr : c.kv.data(),
                                       c.bt.empty() ? nullptr : c.bt.data(), &plan, nullptr);
  CHECK(s == want, "%s: status %d, want %d (%s)", c.name.c_str(), int(s), int(want), varlen_attn_last_error());
  CHECK(plan == nullptr && varlen_attn_last_error()[0] != 0, "%s: refused plan", c.name.c_str());
}

}  // namespace

int main() {
  std::mt19937_64 rng(2024);
  int64_t outputs = 0;
  // ---- refused metadata
  {
    Case ok = make("valid", {3, 1}, {10, 40}, 4, 2, 64, 16, VA_DTYPE_BF16, rng);
    auto bad = [&](const std::string& name, auto edit, va_status want) {
      Case c = ok;
      c.name = name;
      edit(c);
      expect_refused(c, want);
    };
    bad("hq % hkv", [](Case& c) { c.p.num_q_heads = 3; }, VA_ERR_INVALID_ARG);
    bad("head_dim 96", [](Case& c) { c.p.head_dim = 96; }, VA_ERR_UNSUPPORTED);
    bad("page 48", [](Case& c) { c.p.page_size = 48; }, VA_ERR_UNSUPPORTED);
    bad("dtype 7", [](Case& c) { c.p.dtype = 7; }, VA_ERR_INVALID_ARG);
    bad("q_rows > kv_len", [](Case& c) { c.qe[0] = c.qs[0] + 11; c.qs[1] += 8; c.qe[1] += 8; }, VA_ERR_INVALID_ARG);
    bad("q_end < q_start", [](Case& c) { c.qe[1] = c.qs[1] - 1; }, VA_ERR_INVALID_ARG);
    bad("overlapping rows", [](Case& c) { c.qs[1] = 2; c.qe[1] = 3; }, VA_ERR_INVALID_ARG);
    bad("page out of range", [](Case& c) { c.bt[0] = c.p.num_pages; }, VA_ERR_INVALID_ARG);
    bad("negative page", [](Case& c) { c.bt[1 * c.p.max_pages_per_req + 1] = -1; }, VA_ERR_INVALID_ARG);
    bad("kv beyond table", [](Case& c) { c.kv[1] = c.p.max_pages_per_req * c.p.page_size + 1; }, VA_ERR_INVALID_ARG);
    bad("no pages", [](Case& c) { c.p.num_pages = 0; }, VA_ERR_INVALID_ARG);
    bad("null metadata", [](Case& c) { c.qs.clear(); }, VA_ERR_INVALID_ARG);
    va_plan* plan = nullptr;
    CHECK(varlen_attn_plan(nullptr, 0, nullptr, nullptr, nullptr, nullptr, &plan, nullptr) == VA_ERR_INVALID_ARG,
          "null params");
    CHECK(varlen_attn_plan(&ok.p, -1, nullptr, nullptr, nullptr, nullptr, &plan, nullptr) == VA_ERR_INVALID_ARG,
          "negative num_reqs");
    varlen_attn_plan_destroy(nullptr);
  }
  // ---- random iterations
  const int ps_opts[] = {16, 32, 64, 128, 256};
  const int dtypes[] = {VA_DTYPE_BF16, VA_DTYPE_F32, VA_DTYPE_FP8_E4M3};
  for (int n = 0; n < 400; ++n) {
    std::uniform_int_distribution<int> U(0, 1 << 30);
    const int R = 1 + U(rng) % 6, ps = ps_opts[U(rng) % 5], hkv = 1 + U(rng) % 2, g = 1 << (U(rng) % 4);
    const int d = U(rng) % 2 ? 64 : 128, dtype = dtypes[U(rng) % 3];
    const bool shared = U(rng) % 4 == 0;
    const int sp = shared ? 1 + U(rng) % 3 : 0;
    std::vector<int> kv, qr;
    for (int r = 0; r < R; ++r) {
      const int k = std::max(sp * ps + 1, 1 + U(rng) % 3000);
      kv.push_back(shared ? std::max(k, sp * ps + ps) : k);
      const int kind = U(rng) % 4;
      const int q = kind == 0 ? 1 : kind == 1 ? 1 + U(rng) % 8 : kind == 2 ? 1 + U(rng) % 300 : kv.back();
      qr.push_back(std::min(q, kv.back()));
    }
    if (shared)   // shared pages must be entirely visible: decodes
      for (int& q : qr) q = 1;
    Case c = make("random " + std::to_string(n), qr, kv, hkv * g, hkv, d, ps, dtype, rng, sp, U(rng) % 3);
    if (U(rng) % 2) c.p.flags |= VA_FLAG_SHARED_PREFIX;
    if (U(rng) % 5 == 0) c.p.flags |= VA_FLAG_NO_PREFILL_KERNEL;
    if (U(rng) % 4 == 0) c.p.flags |= VA_FLAG_NO_DECODE_TILES;
    if (U(rng) % 4 == 0) c.p.split_len = 64 * (1 + U(rng) % 16);
    const int cut = U(rng) % 4;
    c.p.prefill_split_len = cut == 0 ? -1 : cut == 1 ? 64 * (1 + U(rng) % 16) : 0;
    if (U(rng) % 5 == 0) c.p.prefill_min_rows = 1 + U(rng) % 64;
    outputs += run_case(c);
  }
  // ---- random tree-shaped sharing: requests point runs of their leading pages at another
  // request's pages (later runs overwrite earlier ones, so runs nest and cross), planned with
  // the shared-prefix flag
  for (int n = 0; n < 300; ++n) {
    std::uniform_int_distribution<int> U(0, 1 << 30);
    const int R = 2 + U(rng) % 24, ps = ps_opts[U(rng) % 5], hkv = 1 + U(rng) % 4, g = 1 << (U(rng) % 4);
    std::vector<int> kv, qr;
    for (int r = 0; r < R; ++r) {
      const int m = U(rng) % 3 == 0 ? 1 + U(rng) % 8 : 1;
      kv.push_back(m + ps * (1 + U(rng) % 24) + U(rng) % ps);
      qr.push_back(m);
    }
    Case c = make("tree-shared " + std::to_string(n), qr, kv, hkv * g, hkv, U(rng) % 2 ? 64 : 128, ps,
                  dtypes[U(rng) % 3], rng);
    const int maxp = c.p.max_pages_per_req;
    const int ops = 1 + U(rng) % 6;
    for (int o = 0; o < ops; ++o) {
      const int src = U(rng) % R;
      for (int r = 0; r < R; ++r) {
        if (r == src || U(rng) % 2) continue;
        // full pages every row of both requests sees
        const int lim = std::min((kv[src] - qr[src] + 1) / ps, (kv[r] - qr[r] + 1) / ps);
        if (lim < 1) continue;
        const int run = 1 + U(rng) % lim;
        for (int j = 0; j < run; ++j) c.bt[size_t(r) * maxp + j] = c.bt[size_t(src) * maxp + j];
      }
    }
    c.p.flags |= VA_FLAG_SHARED_PREFIX;
    if (U(rng) % 4 == 0) c.p.flags |= VA_FLAG_NO_DECODE_TILES;
    if (U(rng) % 5 == 0) c.p.flags |= VA_FLAG_NO_PREFILL_KERNEL;
    outputs += run_case(c);
  }
  // ---- the pages' workload shapes
  {
    std::uniform_int_distribution<int> dec(1024, 8192), mix(512, 16384);
    std::vector<int> kv, q;
    for (int r = 0; r < 256; ++r) kv.push_back(dec(rng)), q.push_back(1);
    outputs += run_case(make("decode-heavy", q, kv, 32, 8, 128, 64, VA_DTYPE_BF16, rng));
    Case nd = make("decode-heavy split items", q, kv, 32, 8, 128, 64, VA_DTYPE_BF16, rng);
    nd.p.flags |= VA_FLAG_NO_DECODE_TILES;
    outputs += run_case(nd);
    std::vector<int> kv4{32768}, q4{2048};
    for (int r = 0; r < 64; ++r) kv4.push_back(mix(rng)), q4.push_back(1);
    outputs += run_case(make("chunk mix", q4, kv4, 64, 8, 128, 64, VA_DTYPE_BF16, rng));
    outputs += run_case(make("orca", {4096, 1, 1}, {4096, 1500, 1700}, 32, 32, 128, 16, VA_DTYPE_BF16, rng));
    std::vector<int> kv9{65536 + 256}, q9{256};
    for (int r = 0; r < 64; ++r) kv9.push_back(mix(rng)), q9.push_back(1);
    outputs += run_case(make("long-prefix chunk", q9, kv9, 32, 8, 128, 64, VA_DTYPE_BF16, rng));
    Case s64 = make("shared-64", std::vector<int>(64, 1), std::vector<int>(64, 17408), 32, 8, 128, 64,
                    VA_DTYPE_BF16, rng, 256);
    s64.p.flags |= VA_FLAG_SHARED_PREFIX;
    outputs += run_case(s64);
    Case s6 = make("shared-6 fp8", std::vector<int>(6, 1), std::vector<int>(6, 5120), 32, 8, 128, 64,
                   VA_DTYPE_FP8_E4M3, rng, 64);
    s6.p.flags |= VA_FLAG_SHARED_PREFIX;
    outputs += run_case(s6);
    std::vector<int> kv7, q7;
    for (int r = 0; r < 256; ++r) kv7.push_back(dec(rng)), q7.push_back(8);
    outputs += run_case(make("8-row verify", q7, kv7, 32, 8, 128, 64, VA_DTYPE_BF16, rng));
    // 128K-context decode: 256 x 131,072 positions, 524,288 block-table entries
    Case lc = make("128K decode", std::vector<int>(256, 1), std::vector<int>(256, 131072), 32, 8, 128, 64,
                   VA_DTYPE_BF16, rng);
    CHECK(lc.bt.size() == 524288, "128K table entries");
    outputs += run_case(lc);
  }
  std::printf("planner sanitized run: %lld outputs checked, %d failures\n", (long long)outputs, g_failures);
  return g_failures ? 1 : 0;
}
