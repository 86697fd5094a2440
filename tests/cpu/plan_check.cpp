// Host-only driver of the GEMM plan's clamp functions (csrc/plan.h): reads
// cases from stdin and prints, for each, what the kernels derive from them.
//   input:  E cap total n  raw_0 .. raw_{E-1}  id_0 .. id_{n-1}
//   output: first_0 rows_0 .. first_{E-1} rows_{E-1}  clamped ids
// Groups are processed as the kernels' scan does: counts clamped to cap, then
// the inclusive prefix S of the clamped counts and first = min(S_excl, total),
// rows = min(S_incl, total) - first.
#include <cstdio>
#include <vector>

#include "../../moe_denoise_forward_amd/csrc/plan.h"

int main() {
  int E, cap, total, n;
  while (std::scanf("%d %d %d %d", &E, &cap, &total, &n) == 4) {
    std::vector<int> raw(E), ids(n);
    for (int& v : raw) std::scanf("%d", &v);
    for (int& v : ids) std::scanf("%d", &v);
    int excl = 0;
    for (int g = 0; g < E; ++g) {
      const int c = plan_clamp_count(raw[g], cap);
      std::printf("%d %d ", plan_first_row(excl, total), plan_rows(excl, excl + c, total));
      excl += c;
    }
    for (int v : ids) std::printf("%d ", plan_clamp_id(v, total));
    std::printf("\n");
  }
  return 0;
}
