// Host-side grouping and work-list construction for IKBO target attention.
//
// Pure C++17 (no HIP): the same file is built into libikbo.so by hipcc and,
// for sanitizer runs, by g++ alone.
//
// The pages give the kernel a candidate-to-user mapping (IKBO blog, section
// 1.3) and let one thread block serve neighbouring candidates of the same
// user (section 3.2, Alg. 1).  Here the mapping is grouped into CSR form once
// on the host, every user's rows are cut into tiles, and the tiles become
// work items (user, head, row tile, key chunk) for a persistent launch.  The
// items are ordered longest-first and dealt to workgroups boustrophedon-style,
// the static jagged load balancing of the Jagged Flash Attention post (TLX
// blog, "scheduling jagged tiles across SMs").
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace ikbo {

// One unit of kernel work.  The layout is read by the device code.
struct WorkItem {
  int32_t kv_base;   // first packed row of the user's K/V (user_offsets[u])
  int32_t row_base;  // target rows: cand_offsets[u]; self rows: user_offsets[u]
  int32_t row0;      // first row of the tile within the user's rows
  int32_t nrows;     // rows in the tile, 1..bm
  int32_t k0, k1;    // key range [k0, k1) within the user's sequence
  int32_t h;         // head
  int32_t kind;      // 0 = target (non-causal), 1 = causal self-attention
  int32_t grp;       // split group, or -1 if the key range is not split
  int32_t chunk;     // index of this key chunk within its group
  int32_t nchunk;    // chunks in the group
  int32_t slot0;     // first partial-result slot of the group
};
static_assert(sizeof(WorkItem) == 48, "WorkItem layout is shared with the kernels");

enum : int32_t { kKindTarget = 0, kKindSelf = 1 };

// Most key chunks one row tile is split into.  Group g owns the partial-result
// slots [g * kMaxSplit, g * kMaxSplit + nchunk), so the merge kernel finds a
// group's slots from its index alone.
constexpr int32_t kMaxSplit = 8;

// One split group (a row tile whose key range was cut into chunks).  Host-side
// description only: the kernels find everything in the partials' row records.
struct MergeItem {
  int32_t row_base, row0, nrows, h, kind, slot0, nchunk, pad;
};

struct PlanParams {
  int32_t bm = 128;           // rows per tile (one workgroup)
  int32_t bn = 64;            // keys per K/V tile; chunk boundaries align to it
  int32_t grid_slots = 512;   // resident workgroups the split decisions assume
  int32_t launch_grid = 0;    // workgroups actually launched (0: grid_slots); never
                              // changes the work list, so results do not depend on it
  int32_t min_chunk = 256;    // shortest key chunk a split may produce
  int32_t max_chunks = kMaxSplit;  // most chunks one key range is cut into (<= kMaxSplit)
  int32_t overhead = 128;     // fixed cost of an item, in key units
  bool allow_split = true;    // split long key ranges (log-sum-exp merge)
  bool single_pass = false;   // split to the shortest chunk length whose items still
                              // fit grid_slots (one item per workgroup), else by cost
  int32_t xcd_bins = 0;       // > 1: multi-pass plans keep all items of one (user, head)
                              // in one of this many bins, one bin per XCD (see HostPlan)
  int32_t group_span = 0;     // > 0, with bins: each bin lists its (user, head) groups in
                              // spans of this many, largest groups first, the items of a
                              // span longest first (for workgroups that take items from a
                              // queue; a static deal needs the whole bin longest first)
  int32_t span_tail = 0;      // with group_span: items of at most this many keys leave
                              // their span for the end of the bin, longest first, so
                              // the bin still ends on its shortest items
};

// Most XCD bins a plan may use (the kernels take the bin offsets by value).
constexpr int32_t kMaxBins = 8;

struct HostPlan {
  std::vector<int32_t> counts;        // [n_users]
  std::vector<int32_t> cand_offsets;  // [n_users + 1]
  std::vector<int32_t> cand_perm;     // [n_cand]
  std::vector<WorkItem> items;        // execution order
  std::vector<MergeItem> groups;      // [n_groups], split groups in group order
  int32_t n_groups = 0;               // split groups
  int32_t n_slots = 0;                // partial-result slots (n_groups * kMaxSplit)
  int32_t grid = 0;                   // workgroups to launch
  int64_t n_target_tiles = 0;
  int64_t n_self_tiles = 0;
  // XCD bins (0 when the plan has none): items [bin_off[b], bin_off[b+1]) are
  // bin b's, each bin longest first (or span by span, see PlanParams::group_span).  Workgroup i of the launch serves bin
  // i % n_bins (the XCD the dispatcher places it on) as its (i / n_bins)-th
  // workgroup, dealing the bin's items boustrophedon-style.  Every item of one
  // (user, head) -- its row tiles, self and target, and key chunks, all reading
  // that user's K/V of that head -- is in one bin, so its re-reads stay in one
  // XCD's L2.  Bins are filled largest (user, head) first, each into the least
  // loaded bin.
  int32_t n_bins = 0;
  int32_t bin_off[kMaxBins + 1] = {};
  // scratch reused by successive builds (no allocation once warm)
  std::vector<int32_t> cursor;
  std::vector<WorkItem> unsorted;
  std::vector<uint64_t> keys;
  std::vector<int64_t> lens;
  std::vector<int64_t> group_cost;
  std::vector<int32_t> group_bin;
};

// Status codes mirror include/ikbo.h.
enum : int {
  kOk = 0, kErrInvalidArg = -1, kErrBadOffsets = -2, kErrBadMapping = -3,
  kErrUnsupported = -4, kErrHip = -5, kErrNoMem = -6
};

// Checks user_offsets (n_users + 1 entries, starts at 0, non-decreasing).
int check_offsets(const int32_t* user_offsets, int32_t n_users, std::string* err);

// CSR grouping.  counts/cand_offsets/cand_perm must hold n_users, n_users + 1
// and n_cand entries.  If tiles is non-null it receives (u, row_start, len)
// triples.  Returns kErrBadMapping for an out-of-range mapping.
int group_csr(const int32_t* cand_to_user, int32_t n_cand, int32_t n_users, int32_t n_q,
              int32_t bm, int32_t* counts, int32_t* cand_offsets, int32_t* cand_perm,
              std::vector<int32_t>* tiles, int64_t* n_tiles, std::string* err,
              std::vector<int32_t>* cursor = nullptr);

// Validates, groups, builds and orders the work list.  Reuses out's storage.
int build_plan(const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users,
               int32_t n_cand, int32_t n_q, int32_t H, bool with_self, const PlanParams& p,
               HostPlan* out, std::string* err);

// Position in the item list of the pass-th item of logical workgroup w when
// `grid` workgroups deal the list boustrophedon-style (even passes left to
// right, odd passes right to left).  Mirrored by the kernels.
inline int64_t zigzag_position(int64_t pass, int32_t w, int32_t grid) {
  return pass * grid + ((pass & 1) ? (grid - 1 - w) : w);
}

}  // namespace ikbo
