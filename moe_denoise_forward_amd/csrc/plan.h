// The clamped expert-major plan of a grouped GEMM launch, as plain integer
// functions (host and device), so the same code is checked on the CPU.
//
// Each GEMM launch derives its tiles from the per-expert pair counts the
// front kernel (or the assign kernel) left in the workspace.  Those counts
// are trusted only within bounds: a count is clamped to [0, cap] (the
// capacity of the expert's pair list), and the experts' rows are fitted,
// in expert order, into the `total` rows that the act / slot buffers hold.
// With S_g the inclusive prefix sum of the clamped counts of experts < g,
// expert g's first row is min(S_g, total) and its row count
// min(S_{g+1}, total) - min(S_g, total): a saturating sum, so the rows of all
// experts never reach past `total`, whatever the counts are.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

__host__ __device__ inline int plan_clamp_count(int raw, int cap) {
  return raw < 0 ? 0 : (raw > cap ? cap : raw);
}

// first row of a group given the exclusive prefix of clamped counts
__host__ __device__ inline int plan_first_row(int excl, int total) { return excl < total ? excl : total; }

// rows of a group given its exclusive and inclusive prefixes
__host__ __device__ inline int plan_rows(int excl, int incl, int total) {
  return plan_first_row(incl, total) - plan_first_row(excl, total);
}

// a row id read from the workspace, clamped into [0, n)
__host__ __device__ inline int plan_clamp_id(int id, int n) {
  return id < 0 ? 0 : (id >= n ? n - 1 : id);
}
