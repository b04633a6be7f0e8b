// Tile table: the n_splits that measured fastest for listed shapes (op, n, D,
// dtype, token range). Written by mhc_hyper_connection_pre_amd/tune.py; the
// library's choice (n_splits = 0) takes an entry that covers the call and is
// valid for it, and its heuristic otherwise.
// Measured on AMD Radeon Graphics (gfx950, 256 CUs) (2026-12-03 12:07 UTC).

#include "mhc_internal.h"

namespace mhc {
namespace {

struct TileEntry {
  int op;               // 0 = mhc_pre, 1 = mhc_post_pre
  int n;
  int64_t D;
  int dt;               // mhc_dtype
  int64_t T_lo, T_hi;   // token counts the entry covers, inclusive
  int n_splits;         // -S: single-pass with S slices; S > 0: two-pass with S splits
};

constexpr TileEntry kTable[] = {
    {0, 4, 4096, 0, 1, 181, -128},
    {0, 4, 4096, 0, 182, 724, -64},
    {0, 4, 4096, 0, 725, 2147483647, -32},
    {1, 4, 4096, 0, 1, 181, -128},
    {1, 4, 4096, 0, 182, 724, -64},
    {1, 4, 4096, 0, 725, 2147483647, -32},
    {0, 4, 5120, 0, 1, 362, -80},
    {0, 4, 5120, 0, 363, 2147483647, -32},
    {1, 4, 5120, 0, 1, 362, -80},
    {1, 4, 5120, 0, 363, 724, -40},
    {1, 4, 5120, 0, 725, 2147483647, -32},
    {0, 4, 7168, 0, 1, 362, -112},
    {0, 4, 7168, 0, 363, 724, -56},
    {0, 4, 7168, 0, 725, 2147483647, -32},
    {1, 4, 7168, 0, 1, 362, -112},
    {1, 4, 7168, 0, 363, 724, -56},
    {1, 4, 7168, 0, 725, 2147483647, -32},
    {-1, 0, 0, 0, 0, 0, 0},   // end
};

}  // namespace

int tuned_splits(int64_t T, int n, int64_t D, mhc_dtype dt, bool boundary) {
  for (const TileEntry& e : kTable) {
    if (e.op == (boundary ? 1 : 0) && e.n == n && e.D == D && e.dt == (int)dt && T >= e.T_lo && T <= e.T_hi)
      return e.n_splits;
  }
  return 0;
}

}  // namespace mhc
