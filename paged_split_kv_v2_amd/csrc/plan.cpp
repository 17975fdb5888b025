// Cascade (shared-prefix) planning and launch, and the chunked-prefix plan.
//
// Cascade [cascade-PR = mlxcel pull request "perf(core): compute shared
// prompt prefixes once per decode batch"]:
//   * "Detection reads the page table, not the refcounts": equal pool rows at
//     equal positions of two page lists are the same bytes, so sharing is
//     found by comparing the host CSR positionally.
//   * "Task items" 1: candidates grouped by first page; each group's span is
//     the longest common page prefix (a member that diverges early shortens
//     the span); the subgroup that removes the most page reads,
//     span * (members - 1), is chosen; one shared level.
//   * "Task items" 2: level 0 is a one-request view over the span; level 1 is
//     the whole batch with the members' span pages removed; non-members keep
//     their whole range and a merge group of one.
//   * "Task items" 4 and "Correctness coverage": shared pages must be full; a
//     span that reaches a member's last page, or is below the page or member
//     threshold, falls back to the flat launch.
//   * "Proving which path a benchmark arm took": the outcome carries batch,
//     members, shared pages/tokens, prefix/suffix chunk counts, or a reason.
// Readings where the page is silent: members ordered by batch index; a span
// equal to a member's page count rejects the group; checks in the order
// member count, span, last page; ties in score go to the lowest first batch
// index; max_groups 0/k extends the single-subgroup rule; the reported
// decline reason is that of the best-scoring rejected group.
//
// Launch layout: every request's partial rows are contiguous,
// [level-0 partitions (members only)][level-1 partitions], so that one
// merge per request equals the page's level merge followed by the pair merge
// (the merge is associative: "How the #898 merge kernel is reused").
//
// Chunked prefix [DCP-PR = ROCm/ATOM pull request "[feat][DCP] Optimize MLA
// DCP ...", section 3.2 figure]: the cached range is cut into chunks, each
// chunk yields (O, LSE), the chunk states are merged, and the result is
// merged with the new-token (suffix) state.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <functional>
#include <map>
#include <vector>

#include "internal.h"
#include "pdk.h"

using namespace pdk;

namespace {

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A set of int32 host arrays uploaded as one blob to the head of a workspace.
struct Blob {
  std::vector<int32_t> data;
  size_t add(const std::vector<int32_t>& v) {
    const size_t off = data.size();
    data.insert(data.end(), v.begin(), v.end());
    while (data.size() % 64) data.push_back(0);  // keep every array 256-byte aligned
    return off;
  }
  size_t bytes() const { return data.size() * sizeof(int32_t); }
};

struct Candidate {
  std::vector<int32_t> members;
  int32_t span;
  long long score;
  int32_t reason;
};

// (view request, partition) pairs of a view, flattened as int pairs, ordered
// by partition length (descending), then request and partition (ascending).
std::vector<int32_t> longest_first(const std::vector<int32_t>& part_indptr,
                                   const std::vector<int32_t>& len, int S) {
  struct Item { int32_t b, p, n; };
  std::vector<Item> items;
  for (size_t b = 0; b + 1 < part_indptr.size(); ++b)
    for (int p = 0; p < part_indptr[b + 1] - part_indptr[b]; ++p)
      items.push_back({(int32_t)b, p, std::max(0, std::min(S, len[b] - p * S))});
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& x, const Item& y) { return x.n > y.n; });
  std::vector<int32_t> out;
  out.reserve(items.size() * 2);
  for (const auto& it : items) {
    out.push_back(it.b);
    out.push_back(it.p);
  }
  return out;
}

}  // namespace

struct pdk_cascade_plan {
  int32_t batch = 0, page_size = 0;
  pdk_cascade_params params{};
  int32_t decline = PDK_DECLINE_NONE;
  int32_t stats[6] = {0, 0, 0, 0, 0, 0};
  std::vector<int32_t> f[PDK_PLAN_NUM_FIELDS];
  // launch bookkeeping
  std::vector<int32_t> l0_part_indptr, l1_part_indptr, member_row_base, l1_row_base;
  int32_t n_groups = 0, n_l0_parts = 0, n_l1_parts = 0, total_rows = 0, max_members = 0;
  Blob blob;
  struct {
    size_t l0_indptr, l0_indices, l0_len, l0_parts, group_indptr, members, member_rows;
    size_t l1_indptr, l1_indices, l1_len, l1_parts, l1_rows, fused;
    size_t l0_work, l1_work, segs;
  } off{};
  const void* uploaded_to = nullptr;
  // page ids of the views live on the device: gathered at upload from these
  // (source offset in the device page ids, workspace int offset, count)
  bool device_views = false;
  int32_t n_segs = 0;
};

extern "C" {

void pdk_cascade_params_default(pdk_cascade_params* p) {
  if (!p) return;
  p->enabled = -1;
  p->min_shared_pages = 16;
  p->min_members = 2;
  p->max_groups = 1;
  p->l0_partition_tokens = 256;
  p->l1_partition_tokens = 512;
  p->fuse_levels = 1;
  p->max_depth = 1;
}

}  // extern "C"

namespace {

int check_params(const pdk_cascade_params& pr, int32_t P) {
  if (pr.min_shared_pages < 1 || pr.min_members < 2 || pr.max_groups < 0)
    return fail(PDK_ERR_ARG, "thresholds: min_shared_pages >= 1, min_members >= 2, max_groups >= 0");
  if (pr.l0_partition_tokens <= 0 || pr.l0_partition_tokens % P ||
      pr.l1_partition_tokens <= 0 || pr.l1_partition_tokens % P)
    return fail(PDK_ERR_ARG, "partition sizes must be positive multiples of page_size %d", P);
  if (pr.fuse_levels != 0 && pr.fuse_levels != 1)
    return fail(PDK_ERR_ARG, "fuse_levels must be 0 or 1");
  if (pr.max_depth < 1) return fail(PDK_ERR_ARG, "max_depth %d < 1", pr.max_depth);
  return PDK_OK;
}

}  // namespace

// The plan from the detection result. leader[b]: the first request (in batch
// order) whose range starts on the same page as b's, or -1 when b has no
// page or no token; common[b]: the number of leading page ids b shares with
// its leader, position by position (a leader's own page count for itself).
// idx: the host page ids, or nullptr when they live only on the device: the
// views' page ids are then gathered there at upload (segments recorded here)
// and nested spans, which compare pages past a span, are not available.
static int upload_blob(pdk_cascade_plan* plan, void* ws, size_t ws_bytes, hipStream_t stream);

// Device detection below a level of spans: for every request b with
// key[b] >= 0 (its span at that level) and off[b] (the span's end page),
// leader[b] is the first request of the same span with the same page at
// off[b] (-1: none) and common[b] the page ids from off[b] it shares with
// that leader, position by position.
typedef std::function<int(const std::vector<int32_t>& key, const std::vector<int32_t>& off,
                          std::vector<int32_t>& leader, std::vector<int32_t>& common)>
    DetectBelow;

static int build_plan(int B, int32_t P, const pdk_cascade_params& pr, const int32_t* indptr,
               const int32_t* len, const int32_t* idx, const std::vector<int32_t>& leader,
               const std::vector<int32_t>& common, pdk_cascade_plan** plan_out,
               const DetectBelow& detect_below = nullptr) {
  auto plan = new pdk_cascade_plan();
  plan->batch = B;
  plan->page_size = P;
  plan->params = pr;
  plan->device_views = idx == nullptr;

  std::vector<Candidate> chosen;
  if (pr.enabled != 1) {
    plan->decline = PDK_DECLINE_DISABLED;
  } else {
    // groups: requests with the same leader (the first member), in order of
    // their leaders; a group's common prefix is the smallest of its members'
    // prefixes shared with the leader
    std::map<int32_t, std::vector<int32_t>> by_leader;
    for (int b = 0; b < B; ++b)
      if (leader[b] >= 0) by_leader[leader[b]].push_back(b);
    std::vector<Candidate> cands;
    for (const auto& kv : by_leader) {
      const auto& mem = kv.second;
      if (mem.size() < 2) continue;
      int32_t lcp = common[mem[0]];
      for (int32_t b : mem) lcp = std::min(lcp, common[b]);
      // every shared page full
      int32_t span = lcp;
      for (int32_t b : mem) span = std::min(span, len[b] / P);
      Candidate c{mem, span, (long long)span * (long long)(mem.size() - 1), PDK_DECLINE_NONE};
      if ((int)mem.size() < pr.min_members) c.reason = PDK_DECLINE_MEMBERS_BELOW_MIN;
      else if (span < pr.min_shared_pages) c.reason = PDK_DECLINE_SPAN_BELOW_MIN;
      else
        for (int32_t b : mem)
          if (span == indptr[b + 1] - indptr[b]) { c.reason = PDK_DECLINE_REACHES_LAST_PAGE; break; }
      cands.push_back(std::move(c));
    }
    auto better = [](const Candidate& x, const Candidate& y) {
      if (x.score != y.score) return x.score > y.score;
      return x.members[0] < y.members[0];
    };
    std::vector<Candidate> ok;
    for (auto& c : cands)
      if (c.reason == PDK_DECLINE_NONE) ok.push_back(c);
    if (cands.empty()) {
      plan->decline = PDK_DECLINE_NO_CANDIDATE;
    } else if (ok.empty()) {
      std::sort(cands.begin(), cands.end(), better);
      plan->decline = cands[0].reason;
    } else {
      std::sort(ok.begin(), ok.end(), better);
      const size_t take = pr.max_groups == 0 ? ok.size() : std::min(ok.size(), (size_t)pr.max_groups);
      chosen.assign(ok.begin(), ok.begin() + take);
      std::sort(chosen.begin(), chosen.end(),
                [](const Candidate& x, const Candidate& y) { return x.members[0] < y.members[0]; });
    }
  }

  // Spans: the selected groups (depth 0), then level by level the child spans
  // of nested sharing: below a span ending at page e, members grouped by
  // their page at e; a subgroup passing the same checks as a group (member
  // count, common prefix from e capped to full pages, span threshold, not
  // reaching a member's last page) is a child span, ordered by first member.
  struct SpanNode {
    std::vector<int32_t> members;
    int32_t start, span, depth, parent;
  };
  std::vector<SpanNode> nodes;
  for (const auto& c : chosen) nodes.push_back({c.members, 0, c.span, 0, -1});
  {
    size_t lo = 0, hi = nodes.size();
    for (int depth = 1; depth < pr.max_depth && (idx || detect_below) && lo < hi; ++depth) {
      std::vector<SpanNode> next;
      // without host page ids: the members' pages at each span's end,
      // grouped and compared on the device
      std::vector<int32_t> lead2, common2;
      if (!idx) {
        std::vector<int32_t> key(B, -1), off(B, -1);
        for (size_t i = lo; i < hi; ++i)
          for (int32_t b : nodes[i].members) {
            key[b] = (int32_t)i;
            off[b] = nodes[i].start + nodes[i].span;
          }
        const int st = detect_below(key, off, lead2, common2);
        if (st) {
          delete plan;
          return st;
        }
      }
      for (size_t i = lo; i < hi; ++i) {
        const int32_t e = nodes[i].start + nodes[i].span;
        // subgroups by the page at e (keyed by page id, or by the subgroup's
        // first member when the device compared them), members ascending
        std::map<int32_t, std::vector<int32_t>> by_page;
        for (int32_t b : nodes[i].members) {
          if (indptr[b + 1] - indptr[b] <= e) continue;
          if (idx) by_page[idx[indptr[b] + e]].push_back(b);
          else if (lead2[b] >= 0) by_page[lead2[b]].push_back(b);
        }
        for (auto& kv : by_page) {
          const auto& mem = kv.second;  // ascending batch order
          if ((int)mem.size() < std::max(2, pr.min_members)) continue;
          // positional common prefix from e of all members
          int32_t c = 0;
          if (idx) {
            for (;;) {
              bool ok = true;
              for (int32_t b : mem)
                if (e + c >= indptr[b + 1] - indptr[b] ||
                    idx[indptr[b] + e + c] != idx[indptr[mem[0]] + e + c]) {
                  ok = false;
                  break;
                }
              if (!ok) break;
              ++c;
            }
          } else {
            // every member's prefix shared with the subgroup's first member
            c = common2[mem[0]];
            for (int32_t b : mem) c = std::min(c, common2[b]);
          }
          for (int32_t b : mem) c = std::min(c, len[b] / P - e);
          if (c < std::max(1, pr.min_shared_pages)) continue;
          bool last = false;
          for (int32_t b : mem) last = last || (e + c == indptr[b + 1] - indptr[b]);
          if (last) continue;
          next.push_back({mem, e, c, depth, (int32_t)i});
        }
      }
      std::sort(next.begin(), next.end(),
                [](const SpanNode& x, const SpanNode& y) { return x.members[0] < y.members[0]; });
      lo = nodes.size();
      nodes.insert(nodes.end(), next.begin(), next.end());
      hi = nodes.size();
    }
  }

  auto& F = plan->f;
  const int K = (int)nodes.size();
  // view page ids (zeros where the device fills them from the segments)
  struct Seg { int32_t src, dst, count; };
  std::vector<int32_t> l0_idx, l1_idx;
  std::vector<Seg> l0_segs, l1_segs;
  plan->n_groups = K;
  std::vector<int32_t> group_of(B, -1), rank(B, -1), private_start(B, 0), n_spans(B, 0);
  F[PDK_PLAN_GROUP_INDPTR].push_back(0);
  F[PDK_PLAN_L0_INDPTR].push_back(0);
  for (int k = 0; k < K; ++k) {
    const auto& c = nodes[k];
    for (size_t m = 0; m < c.members.size(); ++m) {
      const int32_t b = c.members[m];
      if (c.depth == 0) {
        group_of[b] = k;
        rank[b] = (int32_t)m;
      }
      // spans are laid out level by level, so the last one seen is the deepest
      private_start[b] = c.start + c.span;
      ++n_spans[b];
      F[PDK_PLAN_MEMBERS].push_back(b);
    }
    F[PDK_PLAN_GROUP_INDPTR].push_back((int32_t)F[PDK_PLAN_MEMBERS].size());
    F[PDK_PLAN_SPAN_PAGES].push_back(c.span);
    F[PDK_PLAN_SPAN_START].push_back(c.start);
    F[PDK_PLAN_SPAN_PARENT].push_back(c.parent);
    const int b0 = c.members[0];
    if (idx) {
      for (int i = 0; i < c.span; ++i) l0_idx.push_back(idx[indptr[b0] + c.start + i]);
    } else {
      l0_segs.push_back({indptr[b0] + c.start, (int32_t)l0_idx.size(), c.span});
      l0_idx.resize(l0_idx.size() + c.span, 0);
    }
    F[PDK_PLAN_L0_INDPTR].push_back((int32_t)l0_idx.size());
    F[PDK_PLAN_L0_LEN].push_back(c.span * P);
    plan->max_members = std::max(plan->max_members, (int32_t)c.members.size());
  }
  F[PDK_PLAN_L1_INDPTR].push_back(0);
  F[PDK_PLAN_MERGE_INDPTR].push_back(0);
  for (int b = 0; b < B; ++b) {
    const int s = private_start[b];
    if (idx) {
      for (int i = indptr[b] + s; i < indptr[b + 1]; ++i) l1_idx.push_back(idx[i]);
    } else {
      const int n = indptr[b + 1] - indptr[b] - s;
      l1_segs.push_back({indptr[b] + s, (int32_t)l1_idx.size(), n});
      l1_idx.resize(l1_idx.size() + n, 0);
    }
    F[PDK_PLAN_L1_INDPTR].push_back((int32_t)l1_idx.size());
    F[PDK_PLAN_L1_LEN].push_back(len[b] - s * P);
    F[PDK_PLAN_MERGE_INDPTR].push_back(F[PDK_PLAN_MERGE_INDPTR].back() + n_spans[b] + 1);
  }
  F[PDK_PLAN_GROUP_OF] = group_of;
  F[PDK_PLAN_MEMBER_RANK] = rank;
  if (idx) {
    F[PDK_PLAN_L0_INDICES] = l0_idx;
    F[PDK_PLAN_L1_INDICES] = l1_idx;
  }

  // partitions of both levels and the fused row layout
  const int S0 = pr.l0_partition_tokens, S1 = pr.l1_partition_tokens;
  plan->l0_part_indptr.assign(1, 0);
  for (int k = 0; k < K; ++k)
    plan->l0_part_indptr.push_back(plan->l0_part_indptr.back() + ceil_div(F[PDK_PLAN_L0_LEN][k], S0));
  // every request owns at least one level-1 row: an empty range is the
  // state (0, -inf), so its merged output is still written
  plan->l1_part_indptr.assign(1, 0);
  for (int b = 0; b < B; ++b)
    plan->l1_part_indptr.push_back(plan->l1_part_indptr.back() +
                                   std::max(1, ceil_div(F[PDK_PLAN_L1_LEN][b], S1)));
  plan->n_l0_parts = plan->l0_part_indptr.back();
  plan->n_l1_parts = plan->l1_part_indptr.back();
  // each request's rows: one block of partitions per span holding it
  // (outermost first), then its level-1 partitions
  auto& fused = F[PDK_PLAN_FUSED_MERGE_INDPTR];
  fused.assign(1, 0);
  plan->l1_row_base.resize(B);
  std::vector<int32_t> next_row(B);
  std::vector<int32_t> span_rows(B, 0);
  for (int k = 0; k < K; ++k)
    for (int32_t b : nodes[k].members)
      span_rows[b] += plan->l0_part_indptr[k + 1] - plan->l0_part_indptr[k];
  for (int b = 0; b < B; ++b) {
    const int n1 = plan->l1_part_indptr[b + 1] - plan->l1_part_indptr[b];
    next_row[b] = fused.back();
    plan->l1_row_base[b] = fused.back() + span_rows[b];
    fused.push_back(fused.back() + span_rows[b] + n1);
  }
  plan->total_rows = fused.back();
  plan->member_row_base.clear();
  for (int k = 0; k < K; ++k)
    for (int32_t b : nodes[k].members) {
      plan->member_row_base.push_back(next_row[b]);
      next_row[b] += plan->l0_part_indptr[k + 1] - plan->l0_part_indptr[k];
    }

  long long shared = 0, pre_chunks = 0, suf_chunks = 0;
  for (int k = 0; k < K; ++k) {
    shared += F[PDK_PLAN_SPAN_PAGES][k];
    pre_chunks += ceil_div((long long)F[PDK_PLAN_SPAN_PAGES][k] * P, S0);
  }
  for (int b = 0; b < B; ++b) suf_chunks += ceil_div(F[PDK_PLAN_L1_LEN][b], S1);
  int32_t distinct = 0;
  for (int b = 0; b < B; ++b) distinct += n_spans[b] > 0;
  plan->stats[0] = B;
  plan->stats[1] = distinct;
  plan->stats[2] = (int32_t)shared;
  plan->stats[3] = (int32_t)(shared * P);
  plan->stats[4] = (int32_t)pre_chunks;
  plan->stats[5] = (int32_t)suf_chunks;

  // device blob (uploaded to the head of the workspace)
  auto& bl = plan->blob;
  plan->off.l0_indptr = bl.add(F[PDK_PLAN_L0_INDPTR]);
  plan->off.l0_indices = bl.add(l0_idx);
  plan->off.l0_len = bl.add(F[PDK_PLAN_L0_LEN]);
  plan->off.l0_parts = bl.add(plan->l0_part_indptr);
  plan->off.group_indptr = bl.add(F[PDK_PLAN_GROUP_INDPTR]);
  plan->off.members = bl.add(F[PDK_PLAN_MEMBERS]);
  plan->off.member_rows = bl.add(plan->member_row_base);
  plan->off.l1_indptr = bl.add(F[PDK_PLAN_L1_INDPTR]);
  plan->off.l1_indices = bl.add(l1_idx);
  plan->off.l1_len = bl.add(F[PDK_PLAN_L1_LEN]);
  plan->off.l1_parts = bl.add(plan->l1_part_indptr);
  plan->off.l1_rows = bl.add(plan->l1_row_base);
  plan->off.fused = bl.add(fused);
  // work lists, longest partition first: the hardware dispatcher hands out
  // workgroups in order, so the short tail partitions fill the last gaps
  plan->off.l0_work = bl.add(longest_first(plan->l0_part_indptr, F[PDK_PLAN_L0_LEN], S0));
  plan->off.l1_work = bl.add(longest_first(plan->l1_part_indptr, F[PDK_PLAN_L1_LEN], S1));
  if (!idx) {
    std::vector<int32_t> segs;
    for (const auto& g : l0_segs)
      segs.insert(segs.end(), {g.src, (int32_t)plan->off.l0_indices + g.dst, g.count});
    for (const auto& g : l1_segs)
      segs.insert(segs.end(), {g.src, (int32_t)plan->off.l1_indices + g.dst, g.count});
    plan->n_segs = (int32_t)(segs.size() / 3);
    plan->off.segs = bl.add(segs);
  }
  *plan_out = plan;
  return PDK_OK;
}

extern "C" {

int pdk_cascade_plan_create(const pdk_csr* csr, int32_t P, const pdk_cascade_params* params,
                            pdk_cascade_plan** plan_out) {
  if (!plan_out || !params) return fail(PDK_ERR_ARG, "NULL plan_out/params");
  *plan_out = nullptr;
  int st = pdk_validate_csr(csr, P, 0x7FFFFFFF);
  if (st) return st;
  if ((st = check_params(*params, P))) return st;
  const int B = csr->batch;
  const int32_t* indptr = csr->indptr;
  const int32_t* idx = csr->indices;
  const int32_t* len = csr->kv_len;
  // detection on the host: leaders by first page, prefixes shared with them
  std::vector<int32_t> leader(B, -1), common(B, 0);
  std::map<int32_t, int32_t> first_of;
  for (int b = 0; b < B; ++b) {
    const int np = indptr[b + 1] - indptr[b];
    if (np < 1 || len[b] < 1) continue;
    const int32_t L = first_of.emplace(idx[indptr[b]], b).first->second;
    leader[b] = L;
    const int n = std::min(np, indptr[L + 1] - indptr[L]);
    int c = 0;
    while (c < n && idx[indptr[b] + c] == idx[indptr[L] + c]) ++c;
    common[b] = c;
  }
  return build_plan(B, P, *params, indptr, len, idx, leader, common, plan_out);
}

size_t pdk_cascade_device_detect_scratch_bytes(int32_t batch) {
  if (batch < 0) return 0;
  return align256(4 * (size_t)std::max(batch, 1) * sizeof(int32_t));
}

int pdk_cascade_plan_create_device(const pdk_csr* csr_dev, const int32_t* indptr_host,
                                   const int32_t* kv_len_host, int32_t P,
                                   const pdk_cascade_params* params, void* scratch,
                                   size_t scratch_bytes, hipStream_t stream,
                                   pdk_cascade_plan** plan_out) {
  if (!plan_out || !params || !csr_dev || !indptr_host || (csr_dev->batch > 0 && !kv_len_host))
    return fail(PDK_ERR_ARG, "NULL argument");
  *plan_out = nullptr;
  const int B = csr_dev->batch;
  if (B < 0 || csr_dev->nnz < 0) return fail(PDK_ERR_ARG, "batch %d, nnz %d", B, csr_dev->nnz);
  if (P <= 0) return fail(PDK_ERR_ARG, "page_size %d", P);
  int st = check_params(*params, P);
  if (st) return st;
  // the host copies of the row offsets and lengths must describe the device
  // table: every page-id read of the kernels stays inside [0, nnz)
  if (indptr_host[0] != 0 || indptr_host[B] > csr_dev->nnz)
    return fail(PDK_ERR_SHAPE, "indptr[0] = %d, indptr[batch] = %d, nnz = %d", indptr_host[0],
                indptr_host[B], csr_dev->nnz);
  for (int b = 0; b < B; ++b) {
    const int n = indptr_host[b + 1] - indptr_host[b];
    if (n < 0 || kv_len_host[b] < 0 || n != ceil_div(kv_len_host[b], P))
      return fail(PDK_ERR_SHAPE, "request %d: %d pages for %d tokens at page size %d", b, n,
                  kv_len_host[b], P);
  }
  std::vector<int32_t> leader(B, -1), common(B, 0);
  if (B == 0 || params->enabled != 1)
    return build_plan(B, P, *params, indptr_host, kv_len_host, nullptr, leader, common,
                      plan_out);
  if (!csr_dev->indptr || !csr_dev->kv_len || (csr_dev->nnz > 0 && !csr_dev->indices))
    return fail(PDK_ERR_ARG, "NULL device page table");
  if (!scratch || scratch_bytes < pdk_cascade_device_detect_scratch_bytes(B))
    return fail(PDK_ERR_WORKSPACE, "detection scratch %zu bytes < %zu", scratch_bytes,
                pdk_cascade_device_detect_scratch_bytes(B));
  // scratch: leader[B], common[B] (read back with one copy), then the keys
  // and offsets of a level of spans
  int32_t* d_out = (int32_t*)scratch;
  int32_t* d_key = d_out + 2 * (size_t)B;
  int32_t* d_off = d_key + B;
  auto detect = [&](const std::vector<int32_t>* key, const std::vector<int32_t>* off,
                    std::vector<int32_t>& lead, std::vector<int32_t>& comm) {
    hipError_t e = hipSuccess;
    if (key) {
      e = hipMemcpyAsync(d_key, key->data(), B * sizeof(int32_t), hipMemcpyHostToDevice, stream);
      if (e == hipSuccess)
        e = hipMemcpyAsync(d_off, off->data(), B * sizeof(int32_t), hipMemcpyHostToDevice,
                           stream);
      if (e != hipSuccess) return fail(PDK_ERR_HIP, "detection upload: %s", hipGetErrorString(e));
    }
    int rc = launch_detect(csr_dev->indptr, csr_dev->indices, csr_dev->kv_len,
                           key ? d_key : nullptr, key ? d_off : nullptr, B, d_out, d_out + B,
                           stream);
    if (rc) return rc;
    std::vector<int32_t> both(2 * (size_t)B);
    e = hipMemcpyAsync(both.data(), d_out, both.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                       stream);
    // also orders the key/offset uploads before their host buffers go away
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(PDK_ERR_HIP, "detection readback: %s", hipGetErrorString(e));
    lead.assign(both.begin(), both.begin() + B);
    comm.assign(both.begin() + B, both.end());
    return (int)PDK_OK;
  };
  if ((st = detect(nullptr, nullptr, leader, common))) return st;
  // nested spans: one more detection per level below the outermost spans
  const DetectBelow below = [&](const std::vector<int32_t>& key, const std::vector<int32_t>& off,
                                std::vector<int32_t>& lead, std::vector<int32_t>& comm) {
    return detect(&key, &off, lead, comm);
  };
  return build_plan(B, P, *params, indptr_host, kv_len_host, nullptr, leader, common, plan_out,
                    below);
}

int pdk_cascade_plan_upload_device(pdk_cascade_plan* plan, const pdk_csr* csr_dev, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  if (!plan || !csr_dev) return fail(PDK_ERR_ARG, "NULL plan/csr");
  int st = upload_blob(plan, ws, ws_bytes, stream);
  if (st || !plan->device_views || plan->n_segs == 0) return st;
  if (plan->batch != csr_dev->batch || !csr_dev->indices)
    return fail(PDK_ERR_ARG, "device page table does not match the plan");
  const int32_t* segs = (const int32_t*)ws + plan->off.segs;
  return launch_gather_pages(csr_dev->indices, segs, plan->n_segs, (int32_t*)ws, stream);
}

void pdk_cascade_plan_free(pdk_cascade_plan* plan) { delete plan; }

int pdk_cascade_plan_get(const pdk_cascade_plan* plan, int32_t field, const int32_t** data,
                         int32_t* len) {
  if (!plan || !data || !len) return fail(PDK_ERR_ARG, "NULL argument");
  if (field < 0 || field >= PDK_PLAN_NUM_FIELDS) return fail(PDK_ERR_ARG, "unknown field %d", field);
  *data = plan->f[field].data();
  *len = (int32_t)plan->f[field].size();
  return PDK_OK;
}

int pdk_cascade_plan_stats(const pdk_cascade_plan* plan, int32_t stats[6], int32_t* decline) {
  if (!plan) return fail(PDK_ERR_ARG, "NULL plan");
  if (stats)
    for (int i = 0; i < 6; ++i) stats[i] = plan->stats[i];
  if (decline) *decline = plan->decline;
  return PDK_OK;
}

static size_t cascade_state_offset(const pdk_cascade_plan* plan) { return align256(plan->blob.bytes()); }

size_t pdk_cascade_workspace_bytes(const pdk_cascade_plan* plan, int32_t Hq, int32_t Dv) {
  if (!plan || Hq <= 0 || Dv <= 0) return 0;
  const size_t rows = (size_t)plan->total_rows * Hq;
  return cascade_state_offset(plan) + align256(rows * Dv * sizeof(float)) + rows * sizeof(float);
}

}  // extern "C"

static int upload_blob(pdk_cascade_plan* plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan || !ws) return fail(PDK_ERR_ARG, "NULL plan/workspace");
  if (ws_bytes < plan->blob.bytes())
    return fail(PDK_ERR_WORKSPACE, "workspace %zu bytes < plan %zu", ws_bytes, plan->blob.bytes());
  if (plan->blob.bytes() > 0) {
    hipError_t e = hipMemcpyAsync(ws, plan->blob.data.data(), plan->blob.bytes(),
                                  hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fail(PDK_ERR_HIP, "plan upload: %s", hipGetErrorString(e));
  }
  plan->uploaded_to = ws;
  return PDK_OK;
}

extern "C" {

int pdk_cascade_plan_upload(pdk_cascade_plan* plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (plan && plan->device_views)
    return fail(PDK_ERR_ARG, "plan's page ids live on the device: use pdk_cascade_plan_upload_device");
  return upload_blob(plan, ws, ws_bytes, stream);
}

int pdk_run_cascade_partials(const pdk_cascade_plan* plan, const pdk_kv_pool* pool,
                             const void* q, int32_t q_dtype, int32_t Hq, float sm_scale,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan || !pool || !q || !ws) return fail(PDK_ERR_ARG, "NULL argument");
  if (pool->page_size != plan->page_size)
    return fail(PDK_ERR_SHAPE, "pool page size %d != plan page size %d", pool->page_size,
                plan->page_size);
  if (plan->uploaded_to != ws)
    return fail(PDK_ERR_WORKSPACE, "plan was not uploaded to this workspace");
  const size_t need = pdk_cascade_workspace_bytes(plan, Hq, pool->head_dim_v);
  if (ws_bytes < need) return fail(PDK_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if (Hq <= 0 || Hq % pool->num_kv_heads) return fail(PDK_ERR_SHAPE, "num_q_heads %d", Hq);
  const int32_t* base = (const int32_t*)ws;
  const auto& o = plan->off;
  float* v_part = (float*)((char*)ws + cascade_state_offset(plan));
  float* lse_part = (float*)((char*)v_part + align256((size_t)plan->total_rows * Hq * pool->head_dim_v * 4));
  const int G = Hq / pool->num_kv_heads;

  // level 0: each selected group's span once, members stacked KV-head-major,
  // partials written straight into the members' rows
  PartialArgs a0{}, a1{};
  bool empty0 = true, empty1 = true;
  if (plan->n_l0_parts > 0) {
    pdk_csr v0{base + o.l0_indptr, base + o.l0_indices, base + o.l0_len, plan->n_groups,
               plan->f[PDK_PLAN_L0_INDPTR].back()};
    int st = partial_args(pool, &v0, q, q_dtype, Hq, sm_scale, plan->params.l0_partition_tokens,
                          base + o.l0_parts, plan->n_l0_parts, base + o.group_indptr,
                          base + o.members, plan->max_members, G, base + o.member_rows, v_part,
                          lse_part, reinterpret_cast<const int2*>(base + o.l0_work), &a0, &empty0);
    if (st) return st;
  }
  // level 1: every request's remaining range (the flat batch when declined)
  pdk_csr v1{base + o.l1_indptr, base + o.l1_indices, base + o.l1_len, plan->batch,
             plan->f[PDK_PLAN_L1_INDPTR].back()};
  int st = partial_args(pool, &v1, q, q_dtype, Hq, sm_scale, plan->params.l1_partition_tokens,
                        base + o.l1_parts, plan->n_l1_parts, nullptr, nullptr, 0, G,
                        base + o.l1_rows, v_part, lse_part,
                        reinterpret_cast<const int2*>(base + o.l1_work), &a1, &empty1);
  if (st) return st;
  // the two levels write disjoint rows: one grid when a fused kernel fits
  if (!empty0 && !empty1 && plan->params.fuse_levels) {
    bool handled = false;
    st = launch_cascade_partials(a0, a1, stream, &handled);
    if (st || handled) return st;
  }
  if (!empty0 && (st = launch_partial(a0, stream))) return st;
  return empty1 ? PDK_OK : launch_partial(a1, stream);
}

int pdk_run_cascade_merge(const pdk_cascade_plan* plan, int32_t Hq, int32_t Dv, float* out,
                          float* lse_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan || !out || !ws) return fail(PDK_ERR_ARG, "NULL argument");
  if (plan->uploaded_to != ws)
    return fail(PDK_ERR_WORKSPACE, "plan was not uploaded to this workspace");
  const size_t need = pdk_cascade_workspace_bytes(plan, Hq, Dv);
  if (need == 0 || ws_bytes < need)
    return fail(PDK_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  const int32_t* base = (const int32_t*)ws;
  float* v_part = (float*)((char*)ws + cascade_state_offset(plan));
  float* lse_part = (float*)((char*)v_part + align256((size_t)plan->total_rows * Hq * Dv * 4));
  // one merge per request over its [level-0][level-1] rows
  return pdk_merge_states(v_part, lse_part, plan->total_rows, base + plan->off.fused, plan->batch,
                          Hq, Dv, out, lse_out, stream);
}

int pdk_run_cascade_decode(const pdk_cascade_plan* plan, const pdk_kv_pool* pool, const void* q,
                           int32_t q_dtype, int32_t Hq, float sm_scale, float* out,
                           float* lse_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!out) return fail(PDK_ERR_ARG, "NULL out");
  int st = pdk_run_cascade_partials(plan, pool, q, q_dtype, Hq, sm_scale, ws, ws_bytes, stream);
  if (st) return st;
  return pdk_run_cascade_merge(plan, Hq, pool->head_dim_v, out, lse_out, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Chunked cached prefix + new suffix [DCP-PR, section 3.2 figure]
// ---------------------------------------------------------------------------

}  // extern "C"

struct pdk_chunked_plan {
  int32_t batch = 0, n_chunks = 0, n_pre_parts = 0, n_suf_parts = 0;
  int32_t ch_nnz = 0, suf_nnz = 0;  // page ids of the chunk and suffix views
  int32_t P = 0, C = 0, S = 0, Ps = 0, Ss = 0;
  Blob blob;
  struct {
    size_t ch_indptr, ch_indices, ch_len, ch_parts, ch_slots, ch_owner, req_chunks;
    size_t suf_indptr, suf_indices, suf_len, suf_parts, pair;
    size_t all_req, all_row_ch, all_row_suf;  // one merge over every partial of a request
  } off{};
  const void* uploaded_to = nullptr;
};

namespace {

// byte offsets of the float regions behind the integer blob
struct ChunkedLayout {
  size_t v_pre, l_pre, v_suf, l_suf, v_ch, l_ch, v_pair, l_pair, v_all, l_all, total;
};

ChunkedLayout chunked_layout(const pdk_chunked_plan* p, int Hq, int Dv) {
  ChunkedLayout L{};
  size_t o = align256(p->blob.bytes());
  auto take = [&](size_t rows, size_t width) {
    const size_t at = o;
    o += align256(rows * width * sizeof(float));
    return at;
  };
  L.v_pre = take((size_t)p->n_pre_parts * Hq, Dv);
  L.l_pre = take((size_t)p->n_pre_parts * Hq, 1);
  L.v_suf = take((size_t)p->n_suf_parts * Hq, Dv);
  L.l_suf = take((size_t)p->n_suf_parts * Hq, 1);
  L.v_ch = take((size_t)p->n_chunks * Hq, Dv);
  L.l_ch = take((size_t)p->n_chunks * Hq, 1);
  L.v_pair = take((size_t)2 * p->batch * Hq, Dv);
  L.l_pair = take((size_t)2 * p->batch * Hq, 1);
  L.v_all = take((size_t)(p->n_pre_parts + p->n_suf_parts) * Hq, Dv);
  L.l_all = take((size_t)(p->n_pre_parts + p->n_suf_parts) * Hq, 1);
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

int pdk_chunked_plan_create(const pdk_csr* pre, int32_t P, int32_t C, int32_t S,
                            const pdk_csr* suf, int32_t Ps, int32_t Ss,
                            pdk_chunked_plan** plan_out) {
  if (!plan_out) return fail(PDK_ERR_ARG, "NULL plan_out");
  *plan_out = nullptr;
  int st = pdk_validate_csr(pre, P, 0x7FFFFFFF);
  if (st) return st;
  if ((st = pdk_validate_csr(suf, Ps, 0x7FFFFFFF))) return st;
  if (pre->batch != suf->batch)
    return fail(PDK_ERR_SHAPE, "prefix batch %d != suffix batch %d", pre->batch, suf->batch);
  if (C <= 0 || C % P || S <= 0 || S % P || Ss <= 0 || Ss % Ps)
    return fail(PDK_ERR_ARG, "chunk/partition sizes must be positive multiples of the page sizes");
  auto plan = new pdk_chunked_plan();
  const int B = pre->batch;
  plan->batch = B;
  plan->P = P; plan->C = C; plan->S = S; plan->Ps = Ps; plan->Ss = Ss;
  std::vector<int32_t> ch_indptr{0}, ch_indices, ch_len, ch_parts{0}, ch_slots{0}, owner,
      req_chunks{0}, suf_parts{0}, pair;
  for (int b = 0; b < B; ++b) {
    const int n = pre->kv_len[b];
    const int nch = ceil_div(n, C);
    for (int c = 0; c < nch; ++c) {
      const int a = c * C, e = std::min(n, (c + 1) * C);
      for (int pg = a / P; pg < ceil_div(e, P); ++pg) ch_indices.push_back(pre->indices[pre->indptr[b] + pg]);
      ch_indptr.push_back((int32_t)ch_indices.size());
      ch_len.push_back(e - a);
      ch_parts.push_back(ch_parts.back() + ceil_div(e - a, S));
      ch_slots.push_back((int32_t)owner.size() + 1);
      owner.push_back(b);
    }
    req_chunks.push_back(req_chunks.back() + nch);
    suf_parts.push_back(suf_parts.back() + ceil_div(suf->kv_len[b], Ss));
  }
  for (int b = 0; b <= B; ++b) pair.push_back(2 * b);
  // all partials of request b in one group: its chunk partitions, then its
  // suffix partitions
  std::vector<int32_t> all_req{0}, all_row_ch, all_row_suf;
  for (int b = 0; b < B; ++b) {
    const int base = all_req.back();
    const int c0 = req_chunks[b], c1 = req_chunks[b + 1];
    for (int k = c0; k < c1; ++k) all_row_ch.push_back(base + ch_parts[k] - ch_parts[c0]);
    all_row_suf.push_back(base + ch_parts[c1] - ch_parts[c0]);
    all_req.push_back(base + ch_parts[c1] - ch_parts[c0] + suf_parts[b + 1] - suf_parts[b]);
  }
  plan->n_chunks = (int32_t)owner.size();
  plan->ch_nnz = (int32_t)ch_indices.size();
  plan->suf_nnz = suf->nnz;
  plan->n_pre_parts = ch_parts.back();
  plan->n_suf_parts = suf_parts.back();
  auto& bl = plan->blob;
  plan->off.ch_indptr = bl.add(ch_indptr);
  plan->off.ch_indices = bl.add(ch_indices);
  plan->off.ch_len = bl.add(ch_len);
  plan->off.ch_parts = bl.add(ch_parts);
  plan->off.ch_slots = bl.add(ch_slots);
  plan->off.ch_owner = bl.add(owner);
  plan->off.req_chunks = bl.add(req_chunks);
  plan->off.suf_indptr = bl.add(std::vector<int32_t>(suf->indptr, suf->indptr + B + 1));
  plan->off.suf_indices = bl.add(std::vector<int32_t>(suf->indices, suf->indices + suf->nnz));
  plan->off.suf_len = bl.add(std::vector<int32_t>(suf->kv_len, suf->kv_len + B));
  plan->off.suf_parts = bl.add(suf_parts);
  plan->off.pair = bl.add(pair);
  plan->off.all_req = bl.add(all_req);
  plan->off.all_row_ch = bl.add(all_row_ch);
  plan->off.all_row_suf = bl.add(all_row_suf);
  *plan_out = plan;
  return PDK_OK;
}

void pdk_chunked_plan_free(pdk_chunked_plan* plan) { delete plan; }

int pdk_chunked_plan_counts(const pdk_chunked_plan* plan, int32_t counts[4]) {
  if (!plan || !counts) return fail(PDK_ERR_ARG, "NULL argument");
  counts[0] = plan->batch;
  counts[1] = plan->n_chunks;
  counts[2] = plan->n_pre_parts;
  counts[3] = plan->n_suf_parts;
  return PDK_OK;
}

size_t pdk_chunked_workspace_bytes(const pdk_chunked_plan* plan, int32_t Hq, int32_t Dv) {
  if (!plan || Hq <= 0 || Dv <= 0) return 0;
  return chunked_layout(plan, Hq, Dv).total;
}

int pdk_chunked_plan_upload(pdk_chunked_plan* plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan || !ws) return fail(PDK_ERR_ARG, "NULL plan/workspace");
  if (ws_bytes < plan->blob.bytes())
    return fail(PDK_ERR_WORKSPACE, "workspace %zu bytes < plan %zu", ws_bytes, plan->blob.bytes());
  hipError_t e = hipMemcpyAsync(ws, plan->blob.data.data(), plan->blob.bytes(),
                                hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail(PDK_ERR_HIP, "plan upload: %s", hipGetErrorString(e));
  plan->uploaded_to = ws;
  return PDK_OK;
}

}  // extern "C"

namespace {

// The chunked split for a step of T query tokens per request: the cached
// chunks non-causally, the suffix causally (T = 1: plain decode); the merges
// take the (token, head) pairs as H = T*Hq heads.
int run_chunked(const pdk_chunked_plan* plan, const pdk_kv_pool* pre_pool,
                const pdk_kv_pool* suf_pool, const void* q, int32_t q_dtype, int32_t Hq,
                int32_t T, float sm_scale, float* out, float* lse_out, float* chunk_out,
                float* chunk_lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan || !pre_pool || !suf_pool || !q || !out || !ws) return fail(PDK_ERR_ARG, "NULL argument");
  if (T < 1 || Hq <= 0 || (long long)T * Hq > 0x7FFFFFFF)
    return fail(PDK_ERR_ARG, "q_tokens %d, num_q_heads %d", T, Hq);
  if (plan->uploaded_to != ws)
    return fail(PDK_ERR_WORKSPACE, "plan was not uploaded to this workspace");
  if (pre_pool->page_size != plan->P || suf_pool->page_size != plan->Ps)
    return fail(PDK_ERR_SHAPE, "pool page sizes do not match the plan");
  const int Dv = pre_pool->head_dim_v;
  if (suf_pool->head_dim_v != Dv || suf_pool->head_dim_k != pre_pool->head_dim_k ||
      suf_pool->num_kv_heads != pre_pool->num_kv_heads)
    return fail(PDK_ERR_SHAPE, "prefix and suffix pools disagree on heads or head dims");
  if ((!chunk_out) != (!chunk_lse)) return fail(PDK_ERR_ARG, "chunk_out/chunk_lse: both or neither");
  if (Hq <= 0 || Hq % pre_pool->num_kv_heads) return fail(PDK_ERR_SHAPE, "num_q_heads %d", Hq);
  const int H = T * Hq;
  const ChunkedLayout L = chunked_layout(plan, H, Dv);
  if (ws_bytes < L.total) return fail(PDK_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, L.total);
  const int32_t* base = (const int32_t*)ws;
  const auto& o = plan->off;
  char* w = (char*)ws;
  float* v_ch = chunk_out ? chunk_out : (float*)(w + L.v_ch);
  float* l_ch = chunk_lse ? chunk_lse : (float*)(w + L.l_ch);
  const int G = Hq / pre_pool->num_kv_heads;
  const int B = plan->batch;
  int st;
  if (!chunk_out) {
    // Without the per-chunk states: every partial of a request (chunk
    // partitions, then suffix partitions) is merged by one launch. Merging
    // is associative, so this equals merging within chunks, across chunks
    // and with the suffix, up to f32 rounding.
    float* v_all = (float*)(w + L.v_all);
    float* l_all = (float*)(w + L.l_all);
    if (plan->n_pre_parts > 0) {
      pdk_csr vc{base + o.ch_indptr, base + o.ch_indices, base + o.ch_len, plan->n_chunks,
                 plan->ch_nnz};
      st = partial_rows(pre_pool, &vc, q, q_dtype, Hq, sm_scale, plan->S, base + o.ch_parts,
                        plan->n_pre_parts, base + o.ch_slots, base + o.ch_owner, 1, G,
                        base + o.all_row_ch, v_all, l_all, stream, nullptr, T, 0);
      if (st) return st;
    }
    if (plan->n_suf_parts > 0) {
      pdk_csr vs{base + o.suf_indptr, base + o.suf_indices, base + o.suf_len, B, plan->suf_nnz};
      st = partial_rows(suf_pool, &vs, q, q_dtype, Hq, sm_scale, plan->Ss, base + o.suf_parts,
                        plan->n_suf_parts, nullptr, nullptr, 0, G, base + o.all_row_suf, v_all,
                        l_all, stream, nullptr, T, 1);
      if (st) return st;
    }
    return merge_rows(v_all, l_all, plan->n_pre_parts + plan->n_suf_parts, base + o.all_req, B,
                      H, Dv, out, lse_out, 1, stream);
  }
  // chunk partials: each (request, chunk) is a view request with one member
  if (plan->n_pre_parts > 0) {
    pdk_csr vc{base + o.ch_indptr, base + o.ch_indices, base + o.ch_len, plan->n_chunks,
                 plan->ch_nnz};
    st = partial_rows(pre_pool, &vc, q, q_dtype, Hq, sm_scale, plan->S, base + o.ch_parts,
                      plan->n_pre_parts, base + o.ch_slots, base + o.ch_owner, 1, G,
                      base + o.ch_parts, (float*)(w + L.v_pre), (float*)(w + L.l_pre), stream,
                      nullptr, T, 0);
    if (st) return st;
  }
  // each chunk's (O, LSE)
  st = merge_rows((float*)(w + L.v_pre), (float*)(w + L.l_pre), plan->n_pre_parts, base + o.ch_parts,
                  plan->n_chunks, H, Dv, v_ch, l_ch, 1, stream);
  if (st) return st;
  // across chunks -> even rows of the pair buffer
  st = merge_rows(v_ch, l_ch, plan->n_chunks, base + o.req_chunks, B, H, Dv,
                  (float*)(w + L.v_pair), (float*)(w + L.l_pair), 2, stream);
  if (st) return st;
  // suffix partials and their merge -> odd rows
  if (plan->n_suf_parts > 0) {
    pdk_csr vs{base + o.suf_indptr, base + o.suf_indices, base + o.suf_len, B, plan->suf_nnz};
    st = partial_rows(suf_pool, &vs, q, q_dtype, Hq, sm_scale, plan->Ss, base + o.suf_parts,
                      plan->n_suf_parts, nullptr, nullptr, 0, G, base + o.suf_parts,
                      (float*)(w + L.v_suf), (float*)(w + L.l_suf), stream, nullptr, T, 1);
    if (st) return st;
  }
  st = merge_rows((float*)(w + L.v_suf), (float*)(w + L.l_suf), plan->n_suf_parts,
                  base + o.suf_parts, B, H, Dv, (float*)(w + L.v_pair) + (size_t)H * Dv,
                  (float*)(w + L.l_pair) + H, 2, stream);
  if (st) return st;
  // prefix state with suffix state
  return merge_rows((float*)(w + L.v_pair), (float*)(w + L.l_pair), 2 * B, base + o.pair, B, H,
                    Dv, out, lse_out, 1, stream);
}

}  // namespace

extern "C" {

int pdk_run_chunked_decode(const pdk_chunked_plan* plan, const pdk_kv_pool* pre_pool,
                           const pdk_kv_pool* suf_pool, const void* q, int32_t q_dtype,
                           int32_t Hq, float sm_scale, float* out, float* lse_out,
                           float* chunk_out, float* chunk_lse, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  return run_chunked(plan, pre_pool, suf_pool, q, q_dtype, Hq, 1, sm_scale, out, lse_out,
                     chunk_out, chunk_lse, ws, ws_bytes, stream);
}

int pdk_run_chunked_multi_token(const pdk_chunked_plan* plan, const pdk_kv_pool* pre_pool,
                                const pdk_kv_pool* suf_pool, const void* q, int32_t q_dtype,
                                int32_t Hq, int32_t T, float sm_scale, float* out,
                                float* lse_out, float* chunk_out, float* chunk_lse, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  return run_chunked(plan, pre_pool, suf_pool, q, q_dtype, Hq, T, sm_scale, out, lse_out,
                     chunk_out, chunk_lse, ws, ws_bytes, stream);
}

}  // extern "C"
