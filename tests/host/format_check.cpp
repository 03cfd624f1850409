// Host build of the kernels' format helpers, driven from tests/test_host_format.py.
// Reads "e2m1 <float bits hex>", "e4m3 <float bits hex>", "scale <bmax> <g>" or
// "div <n> <d>" lines on stdin and prints one result per line; "topk <E> <k>
// <E float bits hex>" prints the k selected expert ids of one router row, chosen
// with the top-k kernel's ranking (router_logit, topk_before) one round at a time.
#include <cstdio>
#include <cstring>

#include "nvfp4_common.hpp"
#include "nvfp4_format.hpp"
#include "moe_select.hpp"

int main() {
  char op[16];
  while (std::scanf("%15s", op) == 1) {
    if (!std::strcmp(op, "e2m1")) {
      unsigned b;
      std::scanf("%x", &b);
      std::printf("%u\n", nvfp4::e2m1_encode(nvfp4::u2f(b)));
    } else if (!std::strcmp(op, "e4m3")) {
      unsigned b;
      std::scanf("%x", &b);
      std::printf("%u\n", nvfp4::e4m3_encode(nvfp4::u2f(b)));
    } else if (!std::strcmp(op, "e4m3v")) {
      unsigned c;
      std::scanf("%u", &c);
      std::printf("%08x\n", nvfp4::f2u(nvfp4::e4m3_value(c)));
    } else if (!std::strcmp(op, "scale")) {
      unsigned bm, gb;
      std::scanf("%x %x", &bm, &gb);
      float g = nvfp4::u2f(gb), r;
      unsigned sc = nvfp4::block_scale(nvfp4::u2f(bm), 6.0f * g, g, &r);
      std::printf("%u %08x\n", sc, nvfp4::f2u(r));
    } else if (!std::strcmp(op, "bf16")) {
      unsigned b;
      std::scanf("%x", &b);
      std::printf("%04x\n", nvfp4::float_to_bf16_bits(nvfp4::u2f(b)));
    } else if (!std::strcmp(op, "topk")) {
      unsigned E, k;
      std::scanf("%u %u", &E, &k);
      float v[1024];
      bool open[1024];
      for (unsigned e = 0; e < E && e < 1024; ++e) {
        unsigned b;
        std::scanf("%x", &b);
        v[e] = nvfp4::router_logit(nvfp4::u2f(b));
        open[e] = true;
      }
      for (unsigned j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int32_t be = 0x7FFFFFFF;
        for (unsigned e = 0; e < E; ++e)
          if (open[e] && nvfp4::topk_before(v[e], (int32_t)e, bv, be)) {
            bv = v[e];
            be = (int32_t)e;
          }
        if (be >= 0 && (unsigned)be < E) open[be] = false;
        std::printf(j + 1 < k ? "%d " : "%d\n", be);
      }
    } else if (!std::strcmp(op, "div")) {
      unsigned n, d;
      std::scanf("%u %u", &n, &d);
      std::printf("%u\n", nvfp4::FastDiv(d).div(n));
    }
  }
  return 0;
}
