// Host-side check of the pack kernels' FP8 E4M3FN and BF16 helpers (rq_fp8.hpp): reads
// float64 values as 16-hex-digit bit patterns, one per line, from stdin and prints, per
// value, the floor byte of v, the down and up bytes of |v|, and the bit pattern of
// BF16(v) as a float64; then the value of every finite byte.
#include <cinttypes>
#include <cstdio>
#include <cstring>

#include "rq_fp8.hpp"

int main() {
    char line[64];
    while (std::fgets(line, sizeof line, stdin)) {
        uint64_t bits = 0;
        if (std::sscanf(line, "%" SCNx64, &bits) != 1) continue;
        double v;
        std::memcpy(&v, &bits, 8);
        const double a = v < 0 ? -v : v;
        const double r = rq::bf16_round(v);
        uint64_t rb;
        std::memcpy(&rb, &r, 8);
        std::printf("%02x %02x %02x %016" PRIx64 "\n", rq::e4m3_floor_byte(v), rq::e4m3_down_byte(a),
                    rq::e4m3_up_byte(a), rb);
    }
    for (uint32_t b = 0; b < 256; ++b) {
        if ((b & 0x7F) == 0x7F) continue;
        const double x = rq::e4m3_value(b);
        uint64_t xb;
        std::memcpy(&xb, &x, 8);
        std::printf("byte %02x %016" PRIx64 "\n", b, xb);
    }
    return 0;
}
