// slots_cli.cpp -- host-only driver of slots.h for the CPU tests (built with g++).
// Reads "S W n1 n2 ... " lines on stdin: each line creates a fresh layer with S sink
// and W window slots, appends chunks of n1, n2, ... frames, and after each append
// prints one JSON object with f0, the frame held by each slot and the recache plan.
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "slots.h"

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    int S, W;
    if (!(in >> S >> W)) continue;
    std::vector<int64_t> slot_frame(size_t(S) + W, -1);
    int64_t f0 = 0;
    int n;
    while (in >> n) {
      for (const ll::WriteEntry& e : ll::append_plan(f0, n, S, W)) slot_frame[size_t(e.slot)] = e.frame;
      f0 += n;
      std::cout << "{\"S\":" << S << ",\"W\":" << W << ",\"f0\":" << f0 << ",\"slot_frame\":[";
      for (size_t i = 0; i < slot_frame.size(); ++i) std::cout << (i ? "," : "") << slot_frame[i];
      std::cout << "],\"recache\":[";
      const std::vector<ll::WriteEntry> rp = ll::recache_plan(f0, S, W);
      for (size_t i = 0; i < rp.size(); ++i)
        std::cout << (i ? "," : "") << "[" << rp[i].src << "," << rp[i].slot << "," << rp[i].frame << "]";
      std::cout << "],\"recache_window\":[";
      const std::vector<ll::WriteEntry> wp = ll::recache_window_plan(f0, S, W);
      for (size_t i = 0; i < wp.size(); ++i)
        std::cout << (i ? "," : "") << "[" << wp[i].src << "," << wp[i].slot << "," << wp[i].frame << "]";
      std::cout << "]}\n";
    }
  }
  return 0;
}
