// Host driver for the payload kernels' last-line bounds check (span_fits in
// bounds.h, the same header the kernels include): reads "r0 n cap" triples of
// unsigned 64-bit integers from stdin, prints 1 when the check lets the copy
// through and 0 when it refuses.
#include <cinttypes>
#include <cstdio>

#include "bounds.h"

int main() {
    uint64_t r0, n, cap;
    while (std::scanf("%" SCNu64 " %" SCNu64 " %" SCNu64, &r0, &n, &cap) == 3)
        std::printf("%d\n", a2av::span_fits(r0, n, cap) ? 1 : 0);
    return 0;
}
