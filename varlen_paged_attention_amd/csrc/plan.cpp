// Host-side planner: validates one iteration's metadata and turns it into work lists
// for the HIP kernels.  Plain C++17 (no HIP calls here; the device upload lives in
// kernels.hip), so the planning logic can be exercised without a GPU.
//
// What it plans, from the pages:
//  * Each request is its own diagonal block over the flat Q tensor; no work crosses
//    requests ("一次 forward 怎么塞下很多个 request", section 6.2).
//  * Rows of long new blocks (prefills and prefill chunks) become MFMA prefill tiles;
//    short ones (decode, q_rows = 1, and few-row requests) become split-KV items whose
//    kv range is cut by kv_length so every wavefront gets a similar amount of KV to
//    stream ("ORCA 和 chunked prefill", section 2: decode and prefill in one iteration;
//    section 4: decode is the C = 1 case of a chunk) -- or, on bf16 pools when there are
//    enough of them, prefill tiles too (a decode is a one-row chunk).  Tiles of a few long
//    requests are cut into key chunks merged like split-KV parts.
//  * With VA_FLAG_SHARED_PREFIX, requests whose block tables start with the same
//    physical pages form a group; the shared pages are scored once per group for all of
//    the group's rows, each row keeping its own running max and sum ("How To Scale Your
//    Model 笔记(7-8)", section 3, 物理存一份，不保证从 HBM 只读一次).
#include <algorithm>
#include <chrono>
#include <mutex>
#include <cmath>
#include <cstring>
#include <functional>
#include <map>
#include <new>
#include <numeric>
#include <queue>
#include <tuple>
#include <string>
#include <vector>

#include "va_internal.h"

namespace va {

static std::string& err_slot() {
  static thread_local std::string s;
  return s;
}
void set_error(const std::string& msg) { err_slot() = msg; }
va_status fail(va_status s, const std::string& msg) {
  err_slot() = msg;
  return s;
}

namespace {

struct Block {          // a set of <= 16 query columns scored against one kv range
  int32_t req, kvh;
  int32_t kstart, kend;
  int32_t max_limit, min_limit;
  std::vector<int32_t> outs;   // output ids (q_row * Hq + q_head)
  std::vector<int32_t> limits;
  bool shared;
  bool tile;         // scored by group tiles (MFMA) rather than split items
  bool direct;
  int32_t nchunks;
  int32_t chunk;     // kv positions per item (the last one may be shorter)
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// fp8 plans: decodes (or shared-prefix members' own keys) whose codes and scales take at
// most this many bytes run as tiles in the launch of the plan's other tiles rather than as
// split-KV items in a launch of their own: streaming at about 4.6 instead of 5.6 TB/s then
// costs less than the separate launch and its combine (about 8 us; break-even near 200 MB
// for decodes, below 138 MB for 64 members' private keys)
constexpr int64_t kFp8FoldBytes = int64_t(64) << 20;

// Shared-prefix groups among requests whose block tables start with the same physical page.
// `mem` are those requests; run(a, b) is the number of leading pages requests a and b have
// in common (already capped by the full pages every row of both sees).  Sorted by their page
// sequences, the requests form a tree of common runs (a node: a range of the sorted order
// whose pairs all share `depth` pages; its children split it where neighbours share no more
// than that).  A group is a node's members not already grouped below it, reading the node's
// `depth` pages once for all of them: it saves (members - 1) * depth page reads.  A dynamic
// programme over the tree picks the groups with the largest total saving (the state: how many
// of a subtree's members are left free for a group higher up), so a member that shares one
// page no longer shortens the others' run, and nested prefixes get groups of their own when
// that saves more than one wider, shallower group.  Returns (members, shared pages) pairs.
template <typename RunFn>
std::vector<std::pair<std::vector<int>, int>> prefix_groups(std::vector<int> mem, const std::vector<int>& lim,
                                                            RunFn run_of, const std::function<bool(int, int)>& less) {
  std::vector<std::pair<std::vector<int>, int>> out;
  const int n = int(mem.size());
  if (n < 2) return out;
  std::sort(mem.begin(), mem.end(), less);
  std::vector<int> lcp(n, 0);                           // lcp[i]: pages mem[i-1] and mem[i] share
  for (int i = 1; i < n; ++i) lcp[i] = run_of(mem[i - 1], mem[i]);
  struct Node {
    int lo, hi, depth;
    std::vector<int> kids;                              // child nodes (ranges of the sorted order)
    std::vector<int64_t> best;                          // best[j]: saving with j members left free
    int group_j = -1;                                   // free count grouped here for best[0]
    std::vector<std::vector<int>> pick;                 // pick[k][t]: free members of kid k for total t
  };
  std::vector<Node> nodes;
  std::function<int(int, int)> build = [&](int lo, int hi) -> int {
    const int id = int(nodes.size());
    nodes.push_back(Node{lo, hi, 0, {}, {}, -1, {}});
    if (hi - lo == 1) {
      nodes[id].depth = lim[mem[lo]];
      return id;
    }
    int d = INT32_MAX;
    for (int i = lo + 1; i < hi; ++i) d = std::min(d, lcp[i]);
    nodes[id].depth = d;
    std::vector<int> kids;
    for (int a = lo; a < hi;) {
      int b = a + 1;
      while (b < hi && lcp[b] > d) ++b;
      kids.push_back(build(a, b));
      a = b;
    }
    nodes[id].kids = kids;
    return id;
  };
  constexpr int64_t kNone = INT64_MIN / 4;
  std::function<void(int)> solve = [&](int id) {
    Node& v = nodes[id];
    if (v.hi - v.lo == 1) {
      v.best = {kNone, 0};                              // one request alone is left free
      return;
    }
    std::vector<int64_t> comb = {0};
    for (int k : v.kids) {
      solve(k);
      const std::vector<int64_t>& cb = nodes[k].best;
      std::vector<int64_t> next(comb.size() + cb.size() - 1, kNone);
      std::vector<int> arg(next.size(), -1);
      for (size_t a = 0; a < comb.size(); ++a)
        if (comb[a] != kNone)
          for (size_t c = 0; c < cb.size(); ++c)
            if (cb[c] != kNone && comb[a] + cb[c] > next[a + c]) {
              next[a + c] = comb[a] + cb[c];
              arg[a + c] = int(c);
            }
      nodes[id].pick.push_back(arg);
      comb.swap(next);
    }
    Node& w = nodes[id];
    w.best = comb;
    if (w.depth >= 1)
      for (size_t j = 2; j < comb.size(); ++j)
        if (comb[j] != kNone && comb[j] + int64_t(j - 1) * w.depth > w.best[0]) {
          w.best[0] = comb[j] + int64_t(j - 1) * w.depth;
          w.group_j = int(j);
        }
  };
  // members of node id left free when it ends with j free (groups below are emitted)
  std::function<void(int, int, std::vector<int>&)> assign = [&](int id, int j, std::vector<int>& free_out) {
    const Node& v = nodes[id];
    if (v.hi - v.lo == 1) {
      free_out.push_back(mem[v.lo]);
      return;
    }
    const bool here = j == 0 && v.group_j >= 0;
    int t = here ? v.group_j : j;
    std::vector<int> kid_j(v.kids.size());
    for (int k = int(v.kids.size()) - 1; k >= 0; --k) {
      kid_j[k] = v.pick[k][t];
      t -= kid_j[k];
    }
    std::vector<int> freed;
    for (size_t k = 0; k < v.kids.size(); ++k) assign(v.kids[k], kid_j[k], freed);
    if (here)
      out.push_back({freed, v.depth});
    else
      free_out.insert(free_out.end(), freed.begin(), freed.end());
  };
  const int root = build(0, n);
  solve(root);
  const std::vector<int64_t>& b = nodes[root].best;
  int jbest = 0;
  for (size_t j = 0; j < b.size(); ++j)
    if (b[j] != kNone && (b[jbest] == kNone || b[j] > b[jbest])) jbest = int(j);
  std::vector<int> left;
  if (b[jbest] > 0) assign(root, jbest, left);
  return out;
}

// Launch order of the prefill tiles.  Workgroup i of a launch goes to XCD i % xcds, and each
// XCD has its own L2: tiles that read the same keys (one request's KV head, or one key
// chunk of it for cut tiles) are placed at positions of one XCD so they share its L2,
// with the XCDs' work balanced (a group larger than an XCD's share is spread over
// several); within an XCD, heaviest tiles first so the ragged end of the grid is made of
// short tiles.  When an XCD's list runs out, the remaining positions take the heaviest
// tiles left in the longest list.
// The first tiles of an XCD fill its CUs one slot each, then each CU's second slot, so XCD
// positions c and c + cpx (cpx CUs per XCD) start together on one CU, whose SIMDs their
// waves share: a CU's first two tiles end when their summed work is done.  Positions
// cpx .. 2 cpx - 1 therefore take the lighter half of the first 2 cpx tiles lightest first,
// pairing the heaviest tile with the lightest, so every CU starts with about the same
// work (the ORCA prefill's first pairs summed 84 to 112 steps of 64 keys heaviest first, 98
// each paired, and the launch took 137.3 against 140.0 us).
void order_tiles(std::vector<PrefillTile>& tiles, int xcds, int cpx) {
  const size_t T = tiles.size();
  if (T < 2) return;
  auto work = [](const PrefillTile& t) { return int64_t(t.kv_end) - t.kbeg; };
  auto key = [](const PrefillTile& t) {
    return std::make_tuple(t.req, t.kvh, t.pbase >= 0 || t.flags != 0 ? t.kbeg : -1);
  };
  std::vector<int32_t> idx(T);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) {
    const auto ka = key(tiles[a]), kb = key(tiles[b]);
    if (ka != kb) return ka < kb;
    return work(tiles[a]) > work(tiles[b]);
  });
  int64_t total = 0;
  for (const PrefillTile& t : tiles) total += work(t);
  const int64_t share = std::max<int64_t>(1, ceil_div(total, xcds));
  struct Piece {
    int64_t work;
    size_t b, e;   // range of idx
  };
  std::vector<Piece> pieces;
  for (size_t b = 0; b < T;) {
    size_t e = b;
    Piece pc{0, b, b};
    while (e < T && key(tiles[idx[e]]) == key(tiles[idx[b]])) {
      const int64_t w = work(tiles[idx[e]]);
      if (pc.e > pc.b && pc.work + w > share) {   // close the piece, start the next
        pieces.push_back(pc);
        pc = Piece{0, e, e};
      }
      pc.work += w;
      pc.e = ++e;
    }
    pieces.push_back(pc);
    b = e;
  }
  std::stable_sort(pieces.begin(), pieces.end(), [](const Piece& a, const Piece& b) { return a.work > b.work; });
  std::vector<std::vector<int32_t>> bins(xcds);
  std::vector<int64_t> load(xcds, 0);
  for (const Piece& pc : pieces) {
    const int x = int(std::min_element(load.begin(), load.end()) - load.begin());
    load[x] += pc.work;
    bins[x].insert(bins[x].end(), idx.begin() + pc.b, idx.begin() + pc.e);
  }
  for (auto& bin : bins) {
    std::stable_sort(bin.begin(), bin.end(), [&](int32_t a, int32_t b) { return work(tiles[a]) > work(tiles[b]); });
    if (cpx > 0 && bin.size() >= 2 * size_t(cpx)) std::reverse(bin.begin() + cpx, bin.begin() + 2 * cpx);
  }
  std::vector<PrefillTile> out;
  out.reserve(T);
  std::vector<size_t> pos(xcds, 0);
  for (size_t p = 0; out.size() < T; ++p) {
    int x = int(p % xcds);
    if (pos[x] == bins[x].size()) {
      size_t most = 0;
      for (int y = 0; y < xcds; ++y)
        if (bins[y].size() - pos[y] > most) most = bins[y].size() - pos[y], x = y;
    }
    out.push_back(tiles[bins[x][pos[x]++]]);
  }
  tiles.swap(out);
}


}  // namespace
}  // namespace va

using namespace va;

extern "C" const char* varlen_attn_last_error(void) { return err_slot().c_str(); }

extern "C" const char* varlen_attn_status_string(va_status s) {
  switch (s) {
    case VA_OK: return "ok";
    case VA_ERR_INVALID_ARG: return "invalid argument";
    case VA_ERR_UNSUPPORTED: return "unsupported configuration";
    case VA_ERR_OUT_OF_MEMORY: return "out of memory";
    case VA_ERR_HIP: return "HIP runtime error";
    case VA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
  }
  return "unknown status";
}

extern "C" va_status varlen_attn_plan(const va_params* params, int32_t num_reqs, const int32_t* q_start,
                                      const int32_t* q_end, const int32_t* kv_len,
                                      const int32_t* block_table_host, va_plan** plan_out,
                                      size_t* workspace_bytes_out) {
  auto t0 = std::chrono::steady_clock::now();
  if (!plan_out) return fail(VA_ERR_INVALID_ARG, "plan_out is NULL");
  *plan_out = nullptr;
  if (!params) return fail(VA_ERR_INVALID_ARG, "params is NULL");
  if (num_reqs < 0) return fail(VA_ERR_INVALID_ARG, "num_reqs < 0");
  if (num_reqs > 0 && (!q_start || !q_end || !kv_len || !block_table_host))
    return fail(VA_ERR_INVALID_ARG, "metadata array is NULL");
  const va_params p = *params;
  if (p.num_q_heads < 1 || p.num_kv_heads < 1) return fail(VA_ERR_INVALID_ARG, "head counts must be >= 1");
  if (p.num_q_heads % p.num_kv_heads != 0)
    return fail(VA_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (p.dtype != VA_DTYPE_BF16 && p.dtype != VA_DTYPE_F32 && p.dtype != VA_DTYPE_FP8_E4M3)
    return fail(VA_ERR_INVALID_ARG, "unknown dtype");
  if (p.head_dim != 64 && p.head_dim != 128) return fail(VA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int ps = p.page_size;
  if (ps != 16 && ps != 32 && ps != 64 && ps != 128 && ps != 256)
    return fail(VA_ERR_UNSUPPORTED, "page_size must be 16, 32, 64, 128 or 256");
  if (p.num_pages < 1 || p.max_pages_per_req < 1)
    return fail(VA_ERR_INVALID_ARG, "num_pages and max_pages_per_req must be >= 1");

  const int Hq = p.num_q_heads, Hkv = p.num_kv_heads, D = p.head_dim;
  const int g = Hq / Hkv;
  int64_t total_rows = 0;
  std::vector<std::pair<int32_t, int32_t>> ranges;
  for (int r = 0; r < num_reqs; ++r) {
    const int64_t qs = q_start[r], qe = q_end[r], kv = kv_len[r];
    const std::string who = "request " + std::to_string(r) + ": ";
    if (qs < 0 || qe < qs) return fail(VA_ERR_INVALID_ARG, who + "need 0 <= q_start <= q_end");
    if (kv < 0) return fail(VA_ERR_INVALID_ARG, who + "kv_len < 0");
    const int64_t m = qe - qs;
    if (m > kv) return fail(VA_ERR_INVALID_ARG, who + "q_rows > kv_len (new rows must be in the context)");
    if (kv > int64_t(p.max_pages_per_req) * ps)
      return fail(VA_ERR_INVALID_ARG, who + "kv_len exceeds max_pages_per_req * page_size");
    // every request's pages are checked (the gather entry point reads them all)
    const int64_t npg = ceil_div(kv, ps);
    const int32_t* row = block_table_host + int64_t(r) * p.max_pages_per_req;
    for (int64_t j = 0; j < npg; ++j)
      if (row[j] < 0 || row[j] >= p.num_pages)
        return fail(VA_ERR_INVALID_ARG, who + "block table entry " + std::to_string(j) + " = " +
                                            std::to_string(row[j]) + " outside [0, num_pages)");
    if (m == 0) continue;
    ranges.push_back({int32_t(qs), int32_t(qe)});
    total_rows = std::max(total_rows, qe);
  }
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first < ranges[i - 1].second)
      return fail(VA_ERR_INVALID_ARG, "Q row ranges of two requests overlap");

  va_plan* plan = new (std::nothrow) va_plan();
  if (!plan) return fail(VA_ERR_OUT_OF_MEMORY, "host allocation of the plan failed");
  plan->p = p;
  plan->num_reqs = num_reqs;
  plan->g = g;
  plan->q_start.assign(q_start, q_start + num_reqs);
  plan->q_end.assign(q_end, q_end + num_reqs);
  plan->kv_len.assign(kv_len, kv_len + num_reqs);
  plan->block_table.assign(block_table_host, block_table_host + int64_t(num_reqs) * p.max_pages_per_req);
  plan->kv_offset.resize(num_reqs + 1, 0);
  for (int r = 0; r < num_reqs; ++r) plan->kv_offset[r + 1] = plan->kv_offset[r] + kv_len[r];

  auto bt = [&](int r, int64_t j) { return block_table_host[int64_t(r) * p.max_pages_per_req + j]; };
  // default: a request gets prefill tiles once its new rows fill half a tile's columns
  auto is_prefill = [&](int m) {
    return p.prefill_min_rows > 0 ? m >= p.prefill_min_rows : int64_t(m) * g >= kPrefillCols / 2;
  };
  const bool use_prefill = !(p.flags & VA_FLAG_NO_PREFILL_KERNEL) && prefill_kernel_available(p);
  // the device's shape: resident prefill workgroups and XCDs (a host-only plan assumes a
  // whole MI355X: 256 compute units in 8 XCDs)
  const int cus = (p.flags & VA_FLAG_HOST_ONLY) ? 0 : device_compute_units();
  const int n_cu = cus > 0 ? cus : 256;
  const int slots_wg = kPrefillWgPerCu * n_cu;
  const int xcds = std::max(1, n_cu / kCusPerXcd);

  // ---- classify requests -------------------------------------------------------
  // Requests with enough new rows always get prefill tiles; the others (decodes,
  // speculative-decode verify rows, short chunks) are "short".
  std::vector<int> tile_reqs, short_reqs;
  for (int r = 0; r < num_reqs; ++r) {
    const int m = q_end[r] - q_start[r];
    if (m == 0) continue;
    (use_prefill && is_prefill(m) ? tile_reqs : short_reqs).push_back(r);
  }
  auto add_tiles = [&](std::vector<PrefillTile>& tiles, int r) {
    const int m = q_end[r] - q_start[r];
    const int S0 = kv_len[r] - m;
    const int ncol = m * g;
    for (int kvh = 0; kvh < Hkv; ++kvh)
      for (int c0 = 0; c0 < ncol; c0 += kPrefillCols) {
        PrefillTile t;
        t.req = r;
        t.kvh = kvh;
        t.c0 = c0;
        t.ncols = std::min(kPrefillCols, ncol - c0);
        t.q0 = q_start[r];
        t.S0 = S0;
        t.kv_end = S0 + (c0 + t.ncols - 1) / g + 1;   // one past the last row's last key
        t.kbeg = 0;
        t.pbase = -1;
        t.pstride = 0;
        t.flags = t.group = 0;
        tiles.push_back(t);
      }
  };

  std::vector<int> split_reqs;
  // ---- shared-prefix groups --------------------------------------------------------
  std::vector<int32_t> shared_pages(num_reqs, 0);   // pages read through the group
  std::vector<std::vector<int>> groups;
  if (p.flags & VA_FLAG_SHARED_PREFIX) {
    std::map<int32_t, std::vector<int>> by_first;
    std::vector<int> lim(num_reqs, 0);
    for (int r : short_reqs) {
      const int m = q_end[r] - q_start[r];
      const int S0 = kv_len[r] - m;
      // a shared page must be full and entirely visible to every row of the request
      lim[r] = std::min(kv_len[r] / ps, (S0 + 1) / ps);
      if (lim[r] >= 1) by_first[bt(r, 0)].push_back(r);
    }
    auto run_of = [&](int a, int b) {
      const int cap = std::min(lim[a], lim[b]);
      int c = 0;
      while (c < cap && bt(a, c) == bt(b, c)) ++c;
      return c;
    };
    const std::function<bool(int, int)> less = [&](int a, int b) {
      const int c = run_of(a, b);
      if (c < lim[a] && c < lim[b]) return bt(a, c) < bt(b, c);
      return lim[a] != lim[b] ? lim[a] < lim[b] : a < b;
    };
    for (auto& kvp : by_first) {
      if (kvp.second.size() < 2) continue;
      for (auto& gr : prefix_groups(kvp.second, lim, run_of, less)) {
        for (int r : gr.first) shared_pages[r] = gr.second;
        groups.push_back(gr.first);
      }
    }
  }

  // ---- cut long prefill tiles into key chunks -------------------------------------
  // A tile's time grows with its keys; when a few long tiles are all there is (a short
  // chunk of a long prompt), they would leave most resident slots idle.  Each such tile is
  // then cut into tiles over consecutive key chunks, and the partial results of a column
  // are merged like split-KV parts.  Chunks start at multiples of the chunk length up to
  // S0 + i_first (the last key every column of the tile sees), so every chunk holds at
  // least one visible key for each column; the last chunk runs to the tile's end and
  // absorbs a remainder shorter than a quarter chunk.  Slots are numbered from 0 here and
  // moved past the split-KV ones below.
  //
  // Without a forced chunk length the planner compares greedy schedules of the tiles over
  // the resident slots (the dispatcher hands each next workgroup to the first free slot):
  // whole tiles, and tiles cut into chunks of each power of two from 256 to 8192 keys,
  // each tile costing its keys plus a fixed start-up, chunk tiles also the writing and
  // re-reading of their partial results.  It takes the shortest schedule (a shorter chunk
  // only when its schedule is 5% shorter than the best longer one's) if it beats whole
  // tiles by 10%.  (Power-of-two chunks measured faster than chunks of the same count but
  // other lengths.)
  auto chunks_of = [&](const PrefillTile& t, int64_t Lc) {
    const int64_t seen = int64_t(t.S0) + t.c0 / g + 1;   // keys [0, S0 + i_first] are seen by all
    if (t.kv_end <= 2 * Lc) return int64_t(1);           // short tiles stay whole
    int64_t n = ceil_div(seen, Lc);
    if (n >= 2 && 4 * (seen - (n - 1) * Lc) < Lc) --n;
    return n;
  };
  // cuts `tiles` in place; the chunk tiles' combine rows go to `rows`, their slots (from 0) to `nslots`
  auto cut_tiles = [&](std::vector<PrefillTile>& tiles, std::vector<CombineRow>& rows, int64_t& nslots) {
    if (tiles.empty() || p.prefill_split_len < 0) return;
    int64_t keys_all = 0, longest = 0;
    for (const PrefillTile& t : tiles) {
      keys_all += t.kv_end;
      longest = std::max<int64_t>(longest, t.kv_end);
    }
    int64_t Lc = 0;
    if (p.prefill_split_len > 0) {
      Lc = ceil_div(p.prefill_split_len, kStepKeys) * kStepKeys;
    } else {
      // modelled costs, in keys of one tile: a tile's start (Q load, pipeline fill, the
      // last iteration's drain; small for the few columns of a decode tile) and, for a
      // chunk tile, writing its columns' partials and reading them back in the combine
      // pass (2 * ncols * (D + 2) floats against the 4 * D bytes of K and V one key brings
      // in), weighted 3x.  The weights were fitted to twelve measured workloads (short and
      // long chunks on 4K-131K prefixes, decode batches, tensor- and data-parallel shares):
      // the chosen length is within 6 % of the best measured one on all twelve.
      auto start_cost = [](const PrefillTile& t) { return int64_t(t.ncols >= 64 ? 128 : 16); };
      auto partial_cost = [&](const PrefillTile& t) { return 3 * 2 * int64_t(t.ncols) * (D + 2) / D; };
      auto greedy = [&](std::vector<int64_t>& costs) {
        std::sort(costs.begin(), costs.end(), std::greater<int64_t>());
        std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
        for (int i = 0; i < slots_wg; ++i) free_at.push(0);
        int64_t end = 0;
        for (int64_t c : costs) {
          const int64_t t = free_at.top() + c;
          free_at.pop();
          free_at.push(t);
          end = std::max(end, t);
        }
        return end;
      };
      std::vector<int64_t> costs;
      costs.reserve(tiles.size());
      for (const PrefillTile& t : tiles) costs.push_back(t.kv_end + start_cost(t));
      int64_t best = greedy(costs);
      const int64_t whole_end = best;
      // candidate chunk lengths: powers of two from 256 to 8192 that cut some tile and
      // give at most 16 tiles per resident slot's worth of keys
      for (int64_t cand = 8192; cand >= 256; cand /= 2) {
        if (longest <= 2 * cand) continue;                       // no tile would be cut
        if (keys_all > 16 * slots_wg * cand) break;              // too many chunk tiles
        costs.clear();
        for (const PrefillTile& t : tiles) {
          const int64_t n = chunks_of(t, cand);
          if (n < 2) {
            costs.push_back(t.kv_end + start_cost(t));
          } else {
            const int64_t extra = start_cost(t) + partial_cost(t);
            for (int64_t j = 0; j + 1 < n; ++j) costs.push_back(cand + extra);
            costs.push_back(t.kv_end - (n - 1) * cand + extra);
          }
        }
        const int64_t end = greedy(costs);
        // a shorter chunk must beat the best longer one by 5 %: the model leaves out costs
        // that grow with the number of chunk tiles (the combine's ramp, partials written
        // past L2), and the longer chunk measured faster where the two were within that
        if (Lc == 0 ? end < best : 20 * end < 19 * best) {
          best = end;
          Lc = cand;
        }
      }
      if (10 * best >= 9 * whole_end) Lc = 0;    // cut only for a 10 % shorter schedule
    }
    if (Lc > 0) {
      std::vector<PrefillTile> cut;
      cut.reserve(tiles.size() + size_t(ceil_div(keys_all, Lc)));
      size_t nrows = 0;
      for (const PrefillTile& t : tiles)
        if (chunks_of(t, Lc) >= 2) nrows += size_t(t.ncols);
      rows.reserve(nrows);
      for (const PrefillTile& t : tiles) {
        const int64_t n = chunks_of(t, Lc);
        if (n < 2) {
          cut.push_back(t);
          continue;
        }
        const int64_t base = nslots;
        nslots += int64_t(t.ncols) * n;
        for (int c = 0; c < t.ncols; ++c) {
          CombineRow cr;
          cr.q_row = t.q0 + (t.c0 + c) / g;
          cr.q_head = t.kvh * g + (t.c0 + c) % g;
          cr.pbase = int32_t(base + int64_t(c) * n);
          cr.nparts = int32_t(n);
          rows.push_back(cr);
        }
        for (int64_t j = 0; j < n; ++j) {
          PrefillTile u = t;
          u.kbeg = int32_t(j * Lc);
          u.kv_end = j + 1 < n ? int32_t((j + 1) * Lc) : t.kv_end;
          u.pbase = int32_t(base + j);
          u.pstride = int32_t(n);
          cut.push_back(u);
        }
      }
      tiles.swap(cut);
    }
  };

  // ---- short requests as prefill tiles -----------------------------------------------
  // A short request can also run as prefill tiles (its g * q_rows columns in one tile per
  // KV head, the tile streaming the request's whole KV range through LDS like a prefill).
  // Measured on bf16 pools, that streams KV faster than the split-KV items once the tiles
  // fill the GPU (decode-heavy: 800 vs 850 us; 4-row verify steps: 833 vs 932 us; 128K
  // decodes: 21.1 vs 21.3 ms) but slower when they do not (16 decodes of 2K: 45 vs 28 us)
  // and for fp8 pools, whose tiles widen every code (644 vs 450 us).  So short requests
  // that are not shared-prefix group members become tiles when the plan is bf16, the row
  // classification is the default one, and the tiles (after cutting) fill every resident
  // slot; otherwise they stay split-KV items.  In an fp8 plan that launches prefill tiles
  // anyway, a few decodes ride in that launch as tiles when their KV is small: their slower
  // streaming through the widening tiles (about 4.6 against 5.6 TB/s as items) then costs
  // less than the split-KV launch and its combine (ORCA's two decodes: 173.5 against
  // 181.6 us; the chunk mix's 64 decodes, 1.15 GB, equal either way, stay items).
  std::vector<CombineRow> cut_rows;
  int64_t cut_slots = 0;
  {
    std::vector<int> fold;
    const bool dflt = use_prefill && p.prefill_min_rows <= 0 && !(p.flags & VA_FLAG_NO_DECODE_TILES);
    const bool fp8_fold = p.dtype == VA_DTYPE_FP8_E4M3 && !tile_reqs.empty();
    const bool may_fold = dflt && (p.dtype == VA_DTYPE_BF16 || fp8_fold);
    int64_t fold_pos = 0;                              // kv positions of the folded requests
    if (may_fold)
      for (int r : short_reqs)
        if (shared_pages[r] == 0) {
          fold.push_back(r);
          fold_pos += kv_len[r];
        }
    std::vector<PrefillTile> tiles;
    for (int r : tile_reqs) add_tiles(tiles, r);
    bool folded = false;
    if (!fold.empty()) {
      std::vector<PrefillTile> with = tiles;
      for (int r : fold) add_tiles(with, r);
      std::vector<CombineRow> rows;
      int64_t nslots = 0;
      cut_tiles(with, rows, nslots);
      const int64_t fold_bytes = fold_pos * int64_t(Hkv) * 2 * (int64_t(p.head_dim) + 4);   // fp8 codes + scales
      if (fp8_fold ? fold_bytes <= kFp8FoldBytes : with.size() >= size_t(slots_wg)) {
        plan->tiles.swap(with);
        cut_rows.swap(rows);
        cut_slots = nslots;
        folded = true;
      }
    }
    if (!folded) {
      cut_tiles(tiles, cut_rows, cut_slots);
      plan->tiles.swap(tiles);
    }
    std::vector<char> is_tile(num_reqs, 0);
    for (int r : tile_reqs) is_tile[r] = 1;
    if (folded)
      for (int r : fold) is_tile[r] = 1;
    for (int r : short_reqs)
      if (!is_tile[r]) split_reqs.push_back(r);
  }

  // ---- column blocks ------------------------------------------------------------------
  std::vector<Block> blocks;
  auto add_blocks = [&](const std::vector<std::pair<int, int>>& rowhead,   // (req, local col)
                        int kvh, int32_t kstart, bool shared, int32_t req_for_table, bool tile) {
    // split blocks of a bf16 or fp8 plan take up to 32 columns (two MFMA column blocks per item)
    // when there are more than 16, so the kv range is read once for all of them
    const size_t width = tile ? size_t(kPrefillCols)
                              : (p.dtype != VA_DTYPE_F32 && rowhead.size() > size_t(kSplitCols) ? size_t(2 * kSplitCols)
                                                                                               : size_t(kSplitCols));
    for (size_t b0 = 0; b0 < rowhead.size(); b0 += width) {
      Block B;
      B.req = req_for_table;
      B.kvh = kvh;
      B.kstart = kstart;
      B.shared = shared;
      B.tile = tile;
      B.direct = false;
      B.max_limit = -1;
      B.min_limit = INT32_MAX;
      for (size_t c = b0; c < std::min(rowhead.size(), b0 + width); ++c) {
        const int r = rowhead[c].first, lc = rowhead[c].second;
        const int m = q_end[r] - q_start[r];
        const int i = lc / g, hh = lc % g;
        const int limit = kv_len[r] - m + i;
        B.outs.push_back((q_start[r] + i) * Hq + kvh * g + hh);
        B.limits.push_back(limit);
        B.max_limit = std::max(B.max_limit, limit);
        B.min_limit = std::min(B.min_limit, limit);
      }
      B.kend = B.max_limit + 1;   // group blocks are cut at the shared length by the caller
      blocks.push_back(std::move(B));
    }
  };
  // A group's shared range is scored by MFMA tiles of up to 128 stacked member columns
  // (column-list tiles of the prefill kernel) where that kernel exists, else by split items.
  const bool group_tiles = use_prefill;
  for (auto& mem : groups) {
    const int32_t kend = shared_pages[mem[0]] * ps;
    for (int kvh = 0; kvh < Hkv; ++kvh) {
      std::vector<std::pair<int, int>> rh;
      for (int r : mem)
        for (int lc = 0; lc < (q_end[r] - q_start[r]) * g; ++lc) rh.push_back({r, lc});
      const size_t first = blocks.size();
      add_blocks(rh, kvh, 0, true, mem[0], group_tiles);
      for (size_t b = first; b < blocks.size(); ++b) blocks[b].kend = kend;
    }
  }
  // A group member's own keys after the shared pages: column-list tiles in the same launch
  // as the group tiles, cut into key chunks so that they fill the slots the launch's other
  // tiles leave (below), instead of split-KV items in a launch of their own (64 members:
  // 94 -> 83 us; 6 members: 24.3 -> 17.7 us).  fp8 plans do so, as for their decodes, only
  // when those keys' codes and scales are small (6 members: 25.2 -> 19.9 us; 64 members,
  // 138 MB: 71.3 -> 77.2 us, so they stay items).
  int64_t suffix_pos = 0;
  for (int r : split_reqs)
    if (shared_pages[r] > 0) suffix_pos += kv_len[r] - int64_t(shared_pages[r]) * ps;
  const bool suffix_tiles =
      use_prefill && p.prefill_min_rows <= 0 && !(p.flags & VA_FLAG_NO_DECODE_TILES) &&
      (p.dtype == VA_DTYPE_BF16 ||
       (p.dtype == VA_DTYPE_FP8_E4M3 && suffix_pos * Hkv * 2 * (int64_t(p.head_dim) + 4) <= kFp8FoldBytes));
  for (int r : split_reqs) {
    const int ncol = (q_end[r] - q_start[r]) * g;
    for (int kvh = 0; kvh < Hkv; ++kvh) {
      std::vector<std::pair<int, int>> rh;
      for (int lc = 0; lc < ncol; ++lc) rh.push_back({r, lc});
      add_blocks(rh, kvh, shared_pages[r] * ps, false, r, suffix_tiles && shared_pages[r] > 0);
    }
  }

  // ---- split length: about 8192 items over the whole iteration (fewer, longer ones when
  // there is little work) ---------------------------------------------------------------
  int64_t work = 0, tile_cols = 0, tile_keys = 0;
  for (auto& B : blocks) {
    if (B.tile) {
      if (!B.shared) continue;   // a member's own keys: one tile per 8192 keys
      tile_cols += 1;
      tile_keys = std::max<int64_t>(tile_keys, B.kend - B.kstart);
    } else {
      work += std::max(0, B.kend - B.kstart);
    }
  }
  int64_t L;
  if (p.split_len > 0) {
    L = ceil_div(p.split_len, kStepKeys) * kStepKeys;
  } else {
    L = ceil_div(std::max<int64_t>(1, ceil_div(work, 8192)), kStepKeys) * kStepKeys;
    if (L < 256) {
      // little split work: cut it into enough items to occupy every SIMD (about 2048
      // resident waves) with short items, down to one 64-key step each, so the latency of
      // a few long items does not set the time
      L = std::min<int64_t>(256, ceil_div(std::max<int64_t>(1, ceil_div(work, 2048)), kStepKeys) * kStepKeys);
    }
    L = std::min<int64_t>(L, 8192);
  }
  plan->split_len = int32_t(L);
  // group tiles: key chunks sized for about one tile per two resident workgroups: the
  // members' own keys and the plan's other tiles share the launch, and every chunk writes
  // its columns' partial results for the combine (64 members of a 16K prefix: 512-key
  // chunks 84 us, 1024-key chunks 74 us; 4096-key chunks 108 us, when one group tile
  // outlasts the rest); at least 256 keys
  const int64_t Lt = std::min<int64_t>(
      4096, std::max<int64_t>(256, ceil_div(ceil_div(tile_keys * tile_cols, std::max(1, slots_wg / 2)), kStepKeys) *
                                       kStepKeys));
  // members' own keys: the shortest key chunk (a power of two from 64 keys) with which the
  // member tiles fit in the resident slots the launch's other tiles leave; keys shorter than
  // it stay one tile (64 members of 16K: whole 1024-key tiles, 71 us where 512-key chunks
  // took 74 us; 6 members of 4K: 128-key chunks, 13.2 us where 64- and 256-key chunks took
  // 15.6 and 14.5 us)
  int64_t other_tiles = int64_t(plan->tiles.size()), member_keys = 0;
  for (auto& B : blocks)
    if (B.tile) {
      const int64_t keys = std::max(0, B.kend - B.kstart);
      if (B.shared)
        other_tiles += ceil_div(keys, Lt);
      else
        member_keys += keys;
    }
  const int64_t free_slots = std::max<int64_t>(1, slots_wg - other_tiles);
  int64_t Ls = kStepKeys;
  while (Ls < 8192 && Ls * free_slots < member_keys) Ls *= 2;
  for (auto& B : blocks) {
    const int64_t keys = std::max(0, B.kend - B.kstart);
    B.chunk = int32_t(B.tile ? (B.shared ? Lt : Ls) : L);
    B.nchunks = int32_t(ceil_div(keys, B.chunk));
    if (B.tile && B.nchunks > 1) {
      // every chunk tile starts at a key all its columns see (a column-list tile's columns
      // each need at least one key); the last chunk runs on to the block's end, through the
      // diagonal of a multi-row member
      const int64_t seen = std::max<int64_t>(1, int64_t(B.min_limit) + 1 - B.kstart);
      B.nchunks = int32_t(std::max<int64_t>(1, std::min<int64_t>(B.nchunks, ceil_div(seen, B.chunk))));
    }
  }

  // ---- partial slots: every (row, head) output of the split path that is not written
  // directly (an output whose one part comes from an item that covers only such outputs)
  std::vector<int32_t> nparts(size_t(total_rows) * Hq, 0);
  for (auto& B : blocks)
    for (int32_t o : B.outs) nparts[o] += B.nchunks;
  std::vector<char> needs_slot(nparts.size(), 0);
  for (auto& B : blocks) {
    bool direct = B.nchunks == 1 && !B.tile;
    for (int32_t o : B.outs) direct = direct && nparts[o] == 1;
    B.direct = direct;
    if (!direct)
      for (int32_t o : B.outs) needs_slot[o] = 1;
  }
  std::vector<int32_t> pbase(nparts.size(), -1);
  std::vector<int32_t> shared_n(nparts.size(), 0);   // slots taken by group items
  int64_t slots = 0;
  for (size_t o = 0; o < nparts.size(); ++o)
    if (nparts[o] > 0 && needs_slot[o]) {
      pbase[o] = int32_t(slots);
      slots += nparts[o];
      CombineRow cr;
      cr.q_row = int32_t(o / Hq);
      cr.q_head = int32_t(o % Hq);
      cr.pbase = pbase[o];
      cr.nparts = nparts[o];
      plan->combine.push_back(cr);
    }
  // slots of the cut prefill tiles follow
  for (PrefillTile& t : plan->tiles)
    if (t.pbase >= 0) t.pbase += int32_t(std::min<int64_t>(slots, INT32_MAX));
  plan->combine.reserve(plan->combine.size() + cut_rows.size());
  for (CombineRow cr : cut_rows) {
    cr.pbase += int32_t(std::min<int64_t>(slots, INT32_MAX));
    plan->combine.push_back(cr);
  }
  slots += cut_slots;
  if (slots > INT32_MAX) {
    delete plan;
    return fail(VA_ERR_UNSUPPORTED, "too many partial results for one plan");
  }
  for (auto& B : blocks)
    if (B.shared)
      for (int32_t o : B.outs) shared_n[o] = B.nchunks;

  // ---- emit columns and items ----------------------------------------------------------
  std::vector<SplitItem> shared_items, own_items;
  for (auto& B : blocks) {
    if (B.nchunks == 0) continue;
    if (B.tile) {
      const int32_t col0 = int32_t(plan->cols.size());
      for (size_t c = 0; c < B.outs.size(); ++c) {
        Column C;
        C.q_row = B.outs[c] / Hq;
        C.q_head = B.outs[c] % Hq;
        C.limit = B.limits[c];
        C.pbase = pbase[B.outs[c]];
        plan->cols.push_back(C);
      }
      for (int32_t j = 0; j < B.nchunks; ++j) {
        PrefillTile t;
        t.req = B.req;
        t.kvh = B.kvh;
        t.c0 = col0;
        t.ncols = int32_t(B.outs.size());
        t.q0 = B.shared ? j : shared_n[B.outs[0]] + j;   // partial slot of this chunk
        t.S0 = int32_t(B.kstart + int64_t(j) * B.chunk);
        t.kv_end = j + 1 == B.nchunks ? B.kend : int32_t(std::min<int64_t>(B.kend, B.kstart + int64_t(j + 1) * B.chunk));
        t.kbeg = t.S0;
        t.pbase = -1;
        t.pstride = 0;
        t.flags = kTileColumnList;
        t.group = B.shared ? 1 : 0;
        plan->gtiles.push_back(t);
        plan->tiles.push_back(t);
      }
      continue;
    }
    const int32_t col0 = int32_t(plan->cols.size());
    for (size_t c = 0; c < B.outs.size(); ++c) {
      Column C;
      C.q_row = B.outs[c] / Hq;
      C.q_head = B.outs[c] % Hq;
      C.limit = B.limits[c];
      C.pbase = pbase[B.outs[c]];
      plan->cols.push_back(C);
    }
    for (int32_t j = 0; j < B.nchunks; ++j) {
      SplitItem it;
      it.req = B.req;
      it.kvh = B.kvh;
      it.col0 = col0;
      it.ncols = int32_t(B.outs.size());
      it.k0 = int32_t(B.kstart + int64_t(j) * B.chunk);
      it.k1 = int32_t(std::min<int64_t>(B.kend, B.kstart + int64_t(j + 1) * B.chunk));
      it.slot = B.shared ? j : shared_n[B.outs[0]] + j;
      it.flags = ((B.min_limit < it.k1 - 1) ? kItemMasked : 0) | (B.direct ? kItemDirect : 0);
      (B.shared ? shared_items : own_items).push_back(it);
    }
  }
  // items of more than 16 columns first (their own launch), then group items (each
  // chunk's blocks adjacent), then longest first within each kind
  plan->items = shared_items;
  plan->items.insert(plan->items.end(), own_items.begin(), own_items.end());
  std::stable_sort(plan->items.begin(), plan->items.end(), [](const SplitItem& a, const SplitItem& b) {
    const bool wa = a.ncols > kSplitCols, wb = b.ncols > kSplitCols;
    if (wa != wb) return wa;
    return (a.k1 - a.k0) > (b.k1 - b.k0);
  });
  plan->items_wide = int32_t(std::count_if(plan->items.begin(), plan->items.end(),
                                           [](const SplitItem& it) { return it.ncols > kSplitCols; }));

  // launch order; with only whole tiles every tile runs on the whole-tile kernel, else
  // every tile runs on the kernel that takes all kinds (one launch, so decode tiles, chunk
  // tiles and group tiles share the GPU instead of running one launch after the other)
  order_tiles(plan->tiles, xcds, n_cu / xcds);
  plan->tiles_whole = std::any_of(plan->tiles.begin(), plan->tiles.end(),
                                  [](const PrefillTile& t) { return t.pbase >= 0 || t.flags != 0; })
                          ? 0
                          : int32_t(plan->tiles.size());

  // ---- counters ---------------------------------------------------------------------
  va_plan_stats& st = plan->stats;
  // bytes of one Q / output element, and of one position of one KV head's K and V
  // (fp8: one byte per element plus a float32 scale each for K and V)
  const int64_t elem = p.dtype == VA_DTYPE_F32 ? 4 : 2;
  const int64_t head_pos_bytes = p.dtype == VA_DTYPE_FP8_E4M3 ? 2 * (int64_t(D) + 4) : 2 * int64_t(D) * elem;
  st.num_reqs = num_reqs;
  st.total_q_rows = total_rows;
  st.prefill_tiles = int64_t(plan->tiles.size());
  st.split_items = int64_t(plan->items.size());
  st.shared_items = int64_t(shared_items.size());
  st.shared_groups = int64_t(groups.size());
  st.partial_slots = slots;
  st.combine_rows = int64_t(plan->combine.size());
  std::vector<char>& is_split = plan->is_split;
  is_split.assign(num_reqs, 0);
  for (int r : split_reqs) is_split[r] = 1;
  int64_t pairs = 0, logical_pos = 0, rows = 0, table_entries = 0, pairs_pf = 0, rows_sp = 0;
  for (int r = 0; r < num_reqs; ++r) {
    const int64_t m = q_end[r] - q_start[r];
    if (m == 0) continue;
    const int64_t kv = kv_len[r], S0 = kv - m;
    const int64_t pr = m * S0 + m * (m + 1) / 2;
    pairs += pr;
    if (!is_split[r]) pairs_pf += pr; else rows_sp += m;
    logical_pos += kv;
    rows += m;
    table_entries += ceil_div(kv, ps);
  }
  const int64_t pos_bytes = int64_t(Hkv) * head_pos_bytes;
  plan->pos_bytes = pos_bytes;
  st.prefill_flops = 4.0 * D * Hq * double(pairs_pf);
  st.split_flops = 4.0 * D * Hq * double(pairs - pairs_pf);
  st.split_q_bytes = rows_sp * Hq * D * elem;
  st.shared_tiles = 0;
  st.shared_tile_flops = 0;
  for (const PrefillTile& t : plan->gtiles)
    if (t.group) {                                 // group tiles (every column sees every key)
      ++st.shared_tiles;
      st.shared_tile_flops += 4.0 * D * t.ncols * double(t.kv_end - t.S0);
    }
  // FLOPs of the split-KV items: visible keys of each column in the item's range
  st.split_item_flops = 0;
  for (const SplitItem& it : plan->items)
    for (int32_t c = it.col0; c < it.col0 + it.ncols; ++c)
      st.split_item_flops += 4.0 * D * double(std::max(0, std::min(it.k1, plan->cols[c].limit + 1) - it.k0));
  st.prefill_split_tiles = std::count_if(plan->tiles.begin(), plan->tiles.end(),
                                         [](const PrefillTile& t) { return t.pbase >= 0; });
  st.direct_items = std::count_if(plan->items.begin(), plan->items.end(),
                                  [](const SplitItem& it) { return (it.flags & kItemDirect) != 0; });

  st.visible_pairs = pairs;
  st.flops = 4.0 * D * Hq * double(pairs);
  st.logical_kv_bytes = logical_pos * pos_bytes;
  st.q_bytes = rows * Hq * D * elem;
  st.o_bytes = st.q_bytes;
  st.table_bytes = table_entries * 4;
  plan->ws_ml_off = 0;
  plan->ws_acc_off = size_t(ceil_div(slots * 2 * 4, 256) * 256);
  plan->ws_bytes = plan->ws_acc_off + size_t(ceil_div(slots * D * 4, 256) * 256);
  if (slots == 0) plan->ws_bytes = 0;
  st.workspace_bytes = int64_t(plan->ws_bytes);

  if (!(p.flags & VA_FLAG_HOST_ONLY)) {
    va_status s = upload_plan(plan);
    if (s != VA_OK) {
      delete plan;
      return s;
    }
  }
  st.plan_host_us =
      std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  *plan_out = plan;
  if (workspace_bytes_out) *workspace_bytes_out = plan->ws_bytes;
  return VA_OK;
}

extern "C" va_status varlen_attn_plan_slots(const va_plan* plan, int64_t* out) {
  if (!plan || !out) return fail(VA_ERR_INVALID_ARG, "plan or out is NULL");
  const int64_t rows = plan->stats.total_q_rows;
  for (int64_t t = 0; t < rows; ++t) out[t] = -1;
  const int ps = plan->p.page_size;
  for (int r = 0; r < plan->num_reqs; ++r) {
    const int32_t* row = plan->block_table.data() + int64_t(r) * plan->p.max_pages_per_req;
    const int m = plan->q_end[r] - plan->q_start[r];
    const int S0 = plan->kv_len[r] - m;
    for (int i = 0; i < m; ++i) {
      const int pos = S0 + i;
      out[plan->q_start[r] + i] = int64_t(row[pos / ps]) * ps + pos % ps;
    }
  }
  return VA_OK;
}

// Distinct-position counters.  They walk every block-table entry, so they are computed on
// the first varlen_attn_plan_stats call instead of in the planner (a serving loop that
// plans every iteration does not pay for them).
static void page_counters(const va_plan* plan) {
  const va_params& p = plan->p;
  const int ps = p.page_size;
  va_plan_stats& st = plan->stats;
  auto bt = [&](int r, int64_t j) { return plan->block_table[int64_t(r) * p.max_pages_per_req + j]; };
  // distinct positions read: all requests, and each class (prefill tiles / split items)
  std::vector<int32_t> max_slot(p.num_pages, 0), max_slot_pf(p.num_pages, 0), max_slot_sp(p.num_pages, 0);
  for (int r = 0; r < plan->num_reqs; ++r) {
    if (plan->q_end[r] == plan->q_start[r]) continue;
    const int64_t kv = plan->kv_len[r];
    std::vector<int32_t>& cls = plan->is_split[r] ? max_slot_sp : max_slot_pf;
    for (int64_t j = 0, npg = ceil_div(kv, ps); j < npg; ++j) {
      const int32_t used = int32_t(std::min<int64_t>(ps, kv - j * ps));
      const int32_t page = bt(r, j);
      max_slot[page] = std::max(max_slot[page], used);
      cls[page] = std::max(cls[page], used);
    }
  }
  int64_t phys_pos = 0, phys_pf = 0, phys_sp = 0;
  for (int32_t v : max_slot) phys_pos += v;
  for (int32_t v : max_slot_pf) phys_pf += v;
  for (int32_t v : max_slot_sp) phys_sp += v;
  st.physical_kv_bytes = phys_pos * plan->pos_bytes;
  st.prefill_kv_bytes = phys_pf * plan->pos_bytes;
  st.split_kv_bytes = phys_sp * plan->pos_bytes;
  // distinct positions the split items read (with group tiles, the shared pages are theirs).
  // Every item range starts on a page boundary or right after another item of the same
  // block, so the slots read in one page form one run [lo, hi): per-page bounds suffice.
  std::vector<int32_t> lo(p.num_pages, INT32_MAX), hi(p.num_pages, 0);
  for (const SplitItem& it : plan->items) {
    if (it.kvh != 0) continue;                      // every KV head reads the same positions
    for (int64_t k = it.k0; k < it.k1;) {
      const int64_t j = k / ps, e = std::min<int64_t>(it.k1, (j + 1) * ps);
      const int32_t page = bt(it.req, j);
      lo[page] = std::min<int32_t>(lo[page], int32_t(k - j * ps));
      hi[page] = std::max<int32_t>(hi[page], int32_t(e - j * ps));
      k = e;
    }
  }
  int64_t n = 0;
  for (int32_t pg = 0; pg < p.num_pages; ++pg)
    if (hi[pg] > 0) n += hi[pg] - lo[pg];
  st.split_item_kv_bytes = n * plan->pos_bytes;
}

extern "C" va_status varlen_attn_plan_stats(const va_plan* plan, va_plan_stats* out) {
  if (!plan || !out) return fail(VA_ERR_INVALID_ARG, "plan or out is NULL");
  std::call_once(plan->page_counters_once, page_counters, plan);
  *out = plan->stats;
  return VA_OK;
}

extern "C" va_status varlen_attn_plan_export(const va_plan* plan, int32_t which, const int32_t** data,
                                             int64_t* count, int32_t* ints_per_entry) {
  if (!plan || !data || !count || !ints_per_entry) return fail(VA_ERR_INVALID_ARG, "NULL argument");
  switch (which) {
    case 0:
      *data = reinterpret_cast<const int32_t*>(plan->items.data());
      *count = int64_t(plan->items.size());
      *ints_per_entry = sizeof(SplitItem) / 4;
      return VA_OK;
    case 1:
      *data = reinterpret_cast<const int32_t*>(plan->cols.data());
      *count = int64_t(plan->cols.size());
      *ints_per_entry = sizeof(Column) / 4;
      return VA_OK;
    case 2:
      *data = reinterpret_cast<const int32_t*>(plan->combine.data());
      *count = int64_t(plan->combine.size());
      *ints_per_entry = sizeof(CombineRow) / 4;
      return VA_OK;
    case 3:
      *data = reinterpret_cast<const int32_t*>(plan->tiles.data());
      *count = int64_t(plan->tiles.size());
      *ints_per_entry = sizeof(PrefillTile) / 4;
      return VA_OK;
    case 4:
      *data = reinterpret_cast<const int32_t*>(plan->gtiles.data());
      *count = int64_t(plan->gtiles.size());
      *ints_per_entry = sizeof(PrefillTile) / 4;
      return VA_OK;
  }
  return fail(VA_ERR_INVALID_ARG,
              "which must be 0 (items), 1 (columns), 2 (combine rows), 3 (tiles) or 4 (column-list tiles)");
}

extern "C" void varlen_attn_plan_destroy(va_plan* plan) {
  if (!plan) return;
  free_plan_device(plan);
  delete plan;
}
