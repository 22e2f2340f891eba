// Host driver for tests/test_rounding_host.py: reads float64 values from the
// file argv[1], converts each with the library's float64 -> bf16 rounding
// (dap::f64_to_bf16, compiled here for the host) and writes the 16-bit
// patterns to argv[2]. No GPU is used.
#include <cstdio>
#include <vector>

#include "../../decoder_attention_paged_amd/csrc/dap_internal.h"

int main(int argc, char** argv) {
    if (argc != 3) return 2;
    FILE* in = std::fopen(argv[1], "rb");
    if (!in) return 3;
    std::vector<double> x;
    double v;
    while (std::fread(&v, sizeof v, 1, in) == 1) x.push_back(v);
    std::fclose(in);
    std::vector<uint16_t> out(x.size());
    for (size_t i = 0; i < x.size(); ++i) out[i] = (uint16_t)dap::f64_to_bf16(x[i]);
    FILE* o = std::fopen(argv[2], "wb");
    if (!o) return 4;
    std::fwrite(out.data(), sizeof(uint16_t), out.size(), o);
    std::fclose(o);
    return 0;
}
