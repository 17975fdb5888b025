// Host build of the partial kernels' page-range clamp (rows.h part_range),
// for tests/test_part_range.py: reads "lo hi kv_len nnz S P p" per line and
// prints "page0 start end".
#include <cstdio>

#include "rows.h"

int main() {
  int lo, hi, len, nnz, S, P, p;
  while (std::scanf("%d %d %d %d %d %d %d", &lo, &hi, &len, &nnz, &S, &P, &p) == 7) {
    int indptr[2] = {lo, hi};
    pdk::PartialArgs a{};
    a.indptr = indptr;
    a.kv_len = &len;
    a.nnz = nnz;
    a.S = S;
    a.P = P;
    int page0, start, end;
    pdk::part_range(a, 0, p, page0, start, end);
    std::printf("%d %d %d\n", page0, start, end);
  }
  return 0;
}
