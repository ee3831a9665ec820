// Host build of the kernels' MXFP4 block-exponent rule (rf_mx_scale_exp from
// rf_internal.h): reads float32 values from argv[1], writes one int32
// exponent per value to argv[2].
#include <cstdio>
#include <vector>

#include "rf_internal.h"

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 3;
  std::vector<float> x;
  float v;
  while (std::fread(&v, sizeof(v), 1, f) == 1) x.push_back(v);
  std::fclose(f);
  std::vector<int> e(x.size());
  for (size_t i = 0; i < x.size(); ++i) e[i] = rf_mx_scale_exp(x[i]);
  FILE* g = std::fopen(argv[2], "wb");
  if (!g) return 4;
  std::fwrite(e.data(), sizeof(int), e.size(), g);
  std::fclose(g);
  return 0;
}
