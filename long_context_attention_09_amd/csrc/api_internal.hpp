// Host-side pieces of the C ABI shared by its source files (argument checks,
// workspace plans and launch sequences).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa {
namespace api {

constexpr int64_t kWorkspaceBudget = int64_t(3) << 30;   // index workspace bytes per query block

// Index workspace layout for query blocks of n_qb queries per sequence.
struct IndexPlan {
  int n_qb, n_chunks;
  size_t off_scores, off_hist, off_state, off_ckey, off_ccnt, off_above, off_csel, off_ceqb, off_lin, total;
};

int check_index(const CsaIndexArgs* a);
// The largest query block whose workspace fits `budget` bytes (n_qb = 0: none).
IndexPlan plan_index(const CsaIndexArgs* a, int64_t budget);
// Every query block of a validated call through workspace `ws` laid out by p.
int run_index(const CsaIndexArgs* a, const IndexPlan& p, char* ws, void* stream);

}  // namespace api
}  // namespace csa
