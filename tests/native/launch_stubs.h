// What the launch stand-ins of launch_stubs.cpp record for the driver.
#pragma once

#include <string>

struct StubLog {
  int device = 0;          // the device hipGetDevice reports (0: 256 CUs, else 80)
  std::string calls;       // launches, in order, space-separated
  int spin_max = -1;       // the last indexer launch's poll limit
  int xcd_local = -1;      // the last indexer launch's block layout
};

extern StubLog g_stub;
